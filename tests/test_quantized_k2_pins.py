"""Pins for the 2-bit per-channel key oracle (``oracle/quantized_kv.py``, KIVI
as §4.2 of the blog.tanteng.space page describes it, asymmetric as "KV Cache量化"
of the ybb.press page says): exact codes for exactly representable inputs,
rounding, clamping and the zero-step channel, the half-step error bound, the
bit positions of the tile layout (stated here from the order in which a
wavefront reads them, not from the oracle's formula), a dense brute force over
the dequantised keys, partials, the KV append, the zero point's closed form
(a per-channel shift of the zero points moves every logit of a row by the same
amount, so the output does not change) and the pages' reason for quantising
keys per channel (smaller error than per token on keys with outlier channels).
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import quantized_kv as qk
from paged_kv_cache_365_amd import workloads as wl


def f16(a):
    return np.asarray(a, dtype=np.float16)


def bf16_to_f64(x):
    return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_codes_of_exact_inputs_round_and_clamp():
    z, s = np.float32(-1.25), np.float32(0.25)
    scale = np.full((1, 4), s, np.float32)
    zero = np.full((1, 4), z, np.float32)
    n = np.arange(4)
    cases = {0.0: n, 0.25: n, -0.25: n, 0.75: np.minimum(n + 1, 3), -0.75: np.maximum(n - 1, 0)}
    for frac, want in cases.items():
        k = f16(float(z) + (n + frac) * float(s))[:, None, None] * np.ones((1, 1, 4), np.float16)
        assert np.array_equal(qk.quantize_k2(k, scale, zero, "f16")[:, 0, 0], want), frac
    # exact halves go to the even code: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    k = f16(float(z) + np.array([0.5, 1.5, 2.5]) * float(s))[:, None, None] * np.ones((1, 1, 4), np.float16)
    assert qk.quantize_k2(k, scale, zero, "f16")[:, 0, 0].tolist() == [0, 2, 2]
    # outside [z, z + 3 s] clamps to 0 or 3
    k = f16(float(z) + np.array([-3.0, -100.0, 3.6, 50.0]) * float(s))[:, None, None] * np.ones((1, 1, 4), np.float16)
    assert qk.quantize_k2(k, scale, zero, "f16")[:, 0, 0].tolist() == [0, 0, 3, 3]


def test_zero_step_channel():
    """A constant channel has s = 0: its key is z whatever the code; the code is
    0 at the zero point (0/0), 3 above it and 0 below it."""
    scale = np.zeros((1, 3), np.float32)
    zero = np.full((1, 3), 0.5, np.float32)
    k = f16([[[0.5, 0.75, 0.25]]])
    codes = qk.quantize_k2(k, scale, zero, "f16")
    assert codes[0, 0].tolist() == [0, 3, 0]
    assert (qk.dequantize_k2(codes, scale, zero) == 0.5).all()


def test_each_channel_uses_its_own_scale_and_zero():
    rng = np.random.default_rng(11)
    Hkv, d = 2, 64
    scale = (2.0 ** -rng.integers(2, 6, size=(Hkv, d))).astype(np.float32)
    zero = (rng.integers(-32, 1, size=(Hkv, d)) / 16.0).astype(np.float32)
    n = rng.integers(0, 4, size=(6, Hkv, d))
    exact = zero.astype(np.float64) + n * scale.astype(np.float64)   # <= 7 significant bits
    k = wl.f64_to_storage(exact, "bf16")
    assert np.array_equal(bf16_to_f64(k), exact)
    assert np.array_equal(qk.quantize_k2(k, scale, zero, "bf16"), n.astype(np.uint8))
    assert np.array_equal(qk.dequantize_k2(n.astype(np.uint8), scale, zero), exact)


def test_error_bound_half_a_step():
    rng = np.random.default_rng(12)
    Hkv, d = 2, 128
    scale = rng.uniform(0.1, 1.0, size=(Hkv, d)).astype(np.float32)
    zero = rng.uniform(-3.0, -1.0, size=(Hkv, d)).astype(np.float32)
    u = rng.uniform(0.0, 3.0, size=(80, Hkv, d))
    k = wl.f64_to_storage(zero + u * scale, "f16")
    kf = k.astype(np.float64)
    inside = (kf >= zero) & (kf <= zero.astype(np.float64) + 3 * scale.astype(np.float64))
    err = np.abs(qk.dequantize_k2(qk.quantize_k2(k, scale, zero, "f16"), scale, zero) - kf)
    assert (err[inside] <= (scale.astype(np.float64) * (0.5 + 2.0 ** -20) * np.ones_like(kf))[inside]).all()


# -- tile layout -----------------------------------------------------------
def lane_order_words(codes_tok):
    """The words of one token's d channels, built from the order in which a
    wavefront consumes them: lane (group q, token) holds d / 64 words; word w
    feeds matrix steps 2w (h = 0) and 2w + 1 (h = 1) of 32 channels each; for
    step j = 2w + h and i = 0..3, the low half of (word >> 2 (4 h + i)) & 0x30003
    is element 2 i and the high half element 2 i + 1 of the lane's 8 channels
    32 j + 8 q + e.  Returns uint32 [4][d / 64]."""
    d = len(codes_tok)
    words = np.zeros((4, d // 64), np.uint64)
    for q in range(4):
        for w in range(d // 64):
            for h in range(2):
                j = 2 * w + h
                for i in range(4):
                    lo = 32 * j + 8 * q + 2 * i
                    words[q, w] |= np.uint64(int(codes_tok[lo]) << (2 * (4 * h + i)))
                    words[q, w] |= np.uint64(int(codes_tok[lo + 1]) << (2 * (4 * h + i) + 16))
    return words.astype(np.uint32)


def test_bit_positions_of_named_channels():
    """head_dim 128: token 0 of a 16-token tile; (channel -> byte offset of its
    word in the tile, bit)."""
    d, bs = 128, 16
    cases = {0: (0, 0), 1: (0, 16), 2: (0, 2), 7: (0, 22), 32: (0, 8), 33: (0, 24), 64: (4, 0),
             96: (4, 8), 8: (128, 0), 16: (256, 0), 24: (384, 0), 127: (388, 30)}
    for c, (byte, bit) in cases.items():
        codes = np.zeros((1, 1, d), np.uint8)
        codes[0, 0, c] = 3
        pool = np.zeros(qk.k2_pool_shape(1, 1, d, bs), np.uint32)
        kp, _ = qk.write_kv_k2(pool, np.zeros((1, 1, d, bs), np.float16),
                               np.ones((1, d), np.float32), np.zeros((1, d), np.float32),
                               codes.astype(np.float16), np.zeros((1, 1, d), np.float16),
                               np.array([0]), "f16")
        raw = kp.reshape(-1).view(np.uint8)
        want = np.zeros(bs * d // 4, np.uint8)
        want[byte + bit // 8] = 3 << (bit % 8)
        assert np.array_equal(raw, want), c


@pytest.mark.parametrize("d,bs", [(64, 16), (128, 16), (128, 8)])
def test_write_kv_k2_matches_the_lane_order(d, bs):
    rng = np.random.default_rng(13 + d + bs)
    nb, Hkv, T = 4, 2, 10
    scale = rng.uniform(0.2, 0.6, size=(Hkv, d)).astype(np.float32)
    zero = rng.uniform(-1.5, -0.5, size=(Hkv, d)).astype(np.float32)
    kp = rng.integers(0, 2 ** 32, size=qk.k2_pool_shape(nb, Hkv, d, bs), dtype=np.uint32)
    vp = wl.normal(rng, (nb, Hkv, d, bs), "bf16")
    kn = wl.normal(rng, (T, Hkv, d), "bf16")
    vn = wl.normal(rng, (T, Hkv, d), "bf16")
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[3] = -1
    k2, v2 = qk.write_kv_k2(kp, vp, scale, zero, kn, vn, slots, "bf16")
    codes = qk.quantize_k2(kn, scale, zero, "bf16")
    ke, ve = kp.copy(), vp.copy()
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        b, o = divmod(int(sl), bs)
        for g in range(Hkv):
            ke[b, g, :, o, :] = lane_order_words(codes[i, g])
            ve[b, g, :, o] = vn[i, g]
    assert np.array_equal(k2, ke) and np.array_equal(v2, ve)


# -- attention over the dequantised keys -------------------------------------
def pack_k2(codes, lens, rng, bs, extra_blocks=2):
    """Contiguous codes [B][L][H_kv][d] -> a permuted 2-bit pool and tables (the
    words from ``lane_order_words``); unused words are random."""
    B, Lmax, Hkv, d = codes.shape
    need = [-(-int(L) // bs) for L in lens]
    nb = sum(need) + extra_blocks
    perm = rng.permutation(nb)
    tables = np.full((B, max(max(need), 1)), -1, np.int32)
    pool = rng.integers(0, 2 ** 32, size=qk.k2_pool_shape(nb, Hkv, d, bs), dtype=np.uint32)
    c = 0
    for s in range(B):
        for j in range(need[s]):
            tables[s, j] = perm[c]
            c += 1
        for t in range(int(lens[s])):
            for g in range(Hkv):
                pool[tables[s, t // bs], g, :, t % bs, :] = lane_order_words(codes[s, t, g])
    return pool, tables


def pack_v(V, tables, lens, nb, bs):
    B, Lmax, Hkv, d = V.shape
    vp = wl.nan_fill((nb, Hkv, d, bs), "bf16")
    for s in range(B):
        for t in range(int(lens[s])):
            vp[tables[s, t // bs], :, :, t % bs] = V[s, t]
    return vp


def dense_causal(qd, K, V, scale):
    """qd [T][H_q][d], K, V [L][H_kv][d] (float64): query i at position L - T + i."""
    T, Hq, d = qd.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((T, Hq, d))
    for i in range(T):
        lim = min(max(L - T + 1 + i, 0), L)
        if lim == 0:
            continue
        for h in range(Hq):
            w = softmax(scale * (K[:lim, h // G] @ qd[i, h]))
            out[i, h] = w @ V[:lim, h // G]
    return out


def random_k2_case(rng, B, Lmax, Hkv, G, d, T, dtype="bf16"):
    codes = rng.integers(0, 4, size=(B, Lmax, Hkv, d)).astype(np.uint8)
    scale = rng.uniform(0.3, 0.9, size=(Hkv, d)).astype(np.float32)
    zero = rng.uniform(-1.6, -0.4, size=(Hkv, d)).astype(np.float32)
    V = wl.normal(rng, (B, Lmax, Hkv, d), dtype)
    q = wl.normal(rng, (B, T, Hkv * G, d), dtype)
    return codes, scale, zero, V, q


@pytest.mark.parametrize("T,bs", [(1, 16), (3, 16), (1, 8), (2, 8)])
def test_decode_equals_dense_over_dequantised_keys(T, bs):
    rng = np.random.default_rng(20 + T + bs)
    B, Hkv, G, d = 3, 2, 4, 64
    lens = [T, 21, 50]
    codes, scale, zero, V, q = random_k2_case(rng, B, max(lens), Hkv, G, d, T)
    pool, tables = pack_k2(codes, lens, rng, bs)
    vp = pack_v(V, tables, lens, pool.shape[0], bs)
    got = qk.paged_decode_k2(q, pool, vp, tables, np.array(lens, np.int32), 0.125, scale, zero,
                             "bf16")
    for s in range(B):
        L = lens[s]
        Kd = zero.astype(np.float64) + codes[s, :L].astype(np.float64) * scale.astype(np.float64)
        Vd = bf16_to_f64(V[s, :L])
        qd = bf16_to_f64(q[s])
        np.testing.assert_allclose(got[s], dense_causal(qd, Kd, Vd, 0.125), rtol=0, atol=1e-12)


def test_partials_merge_to_decode():
    from oracle import merge_partials
    rng = np.random.default_rng(21)
    B, Hkv, G, d, T = 2, 2, 2, 128, 2
    lens = [7, 40]
    codes, scale, zero, V, q = random_k2_case(rng, B, 40, Hkv, G, d, T, "f16")
    pool, tables = pack_k2(codes, lens, rng, 16)
    vp = np.zeros((pool.shape[0], Hkv, d, 16), np.float16)
    for s in range(B):
        for t in range(lens[s]):
            vp[tables[s, t // 16], :, :, t % 16] = V[s, t]
    want = qk.paged_decode_k2(q, pool, vp, tables, np.array(lens), 0.1, scale, zero, "f16")
    o, lse = qk.paged_decode_k2_partials(q, pool, vp, tables, np.array(lens), 0.1, scale, zero,
                                         "f16", 16, 40)
    np.testing.assert_allclose(merge_partials(o, lse).reshape(want.shape), want, rtol=0, atol=1e-13)


def test_zero_point_shift_leaves_the_output():
    """k_hat = z + s code: shifting z by delta_c moves every logit of a row by
    scale * q . delta, the same for all tokens, so softmax and output stay."""
    rng = np.random.default_rng(22)
    B, Hkv, G, d, T = 2, 2, 4, 64, 1
    lens = [33, 18]
    codes, scale, zero, V, q = random_k2_case(rng, B, 33, Hkv, G, d, T)
    pool, tables = pack_k2(codes, lens, rng, 16)
    vp = pack_v(V, tables, lens, pool.shape[0], 16)
    a = qk.paged_decode_k2(q, pool, vp, tables, np.array(lens), 0.125, scale, zero, "bf16")
    shifted = (zero + rng.uniform(-4, 4, size=zero.shape)).astype(np.float32)
    b = qk.paged_decode_k2(q, pool, vp, tables, np.array(lens), 0.125, scale, shifted, "bf16")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # every step zero: all keys equal their zero point, weights are uniform
    c = qk.paged_decode_k2(q, pool, vp, tables, np.array(lens), 0.125, np.zeros_like(scale), zero,
                           "bf16")
    for s in range(B):
        mean_v = bf16_to_f64(V[s, :lens[s]]).mean(axis=0)                # [H_kv][d]
        np.testing.assert_allclose(c[s, 0], np.repeat(mean_v, G, axis=0), rtol=0, atol=1e-12)


def test_per_channel_beats_per_token_on_outlier_channels():
    """§4.2 of the blog.tanteng.space page: per-token 2-bit key quantisation has a
    large error, per-channel a small one.  Keys with a few channels 10x the rest:
    the per-token range is set by the outliers and the other channels lose their
    information."""
    rng = np.random.default_rng(5)
    L, d = 512, 128
    K = rng.standard_normal((L, 1, d))
    K[:, 0, rng.choice(d, 4, replace=False)] *= 10.0
    Kb = wl.f64_to_storage(K, "bf16")
    Kf = bf16_to_f64(Kb)
    lo, hi = Kf.min(axis=0), Kf.max(axis=0)                   # per channel [1][d]
    s_c, z_c = ((hi - lo) / 3).astype(np.float32), lo.astype(np.float32)
    err_channel = np.mean((qk.dequantize_k2(qk.quantize_k2(Kb, s_c, z_c, "bf16"), s_c, z_c) - Kf) ** 2)
    lo_t, hi_t = Kf.min(axis=2, keepdims=True), Kf.max(axis=2, keepdims=True)  # per token
    s_t = np.broadcast_to((hi_t - lo_t) / 3, Kf.shape).astype(np.float32)
    z_t = np.broadcast_to(lo_t, Kf.shape).astype(np.float32)
    err_token = np.mean((qk.dequantize_k2(qk.quantize_k2(Kb, s_t, z_t, "bf16"), s_t, z_t) - Kf) ** 2)
    assert err_token > 2.5 * err_channel


def test_partial_lse_equals_dense_log_sum_exp():
    """The zero point leaves the output but moves each partial's log-sum-exp:
    lse = ln sum_t exp(scale * q . (z + s code_t)) over the partition's tokens,
    computed here densely."""
    rng = np.random.default_rng(23)
    B, Hkv, G, d, T, P = 1, 2, 2, 64, 1, 16
    lens = [37]
    codes, scale, zero, V, q = random_k2_case(rng, B, 37, Hkv, G, d, T)
    pool, tables = pack_k2(codes, lens, rng, 16)
    vp = pack_v(V, tables, lens, pool.shape[0], 16)
    o, lse = qk.paged_decode_k2_partials(q, pool, vp, tables, np.array(lens), 0.125, scale, zero,
                                         "bf16", P, 37)
    Kd = zero.astype(np.float64) + codes[0].astype(np.float64) * scale.astype(np.float64)
    qd = bf16_to_f64(q[0, 0])
    for h in range(Hkv * G):
        x = 0.125 * (Kd[:, h // G] @ qd[h])
        for p in range(3):
            xs = x[p * P:min(37, (p + 1) * P)]
            np.testing.assert_allclose(lse[0, h, p], np.log(np.exp(xs).sum()), rtol=0, atol=1e-12)


def test_calibrated_range_ends_map_to_the_end_codes():
    """The sketch of §4.2 (blog.tanteng.space page) divides a channel's range by
    2^bits - 1: with z = the channel minimum and s = (max - min) / 3, the minimum
    and the maximum of the calibration keys get codes 0 and 3 and dequantise to
    themselves (up to the float32 rounding of s), and the middle of the range
    lies half-way between codes 1 and 2 (rounded to the even one, 2)."""
    rng = np.random.default_rng(30)
    K = wl.f64_to_storage(rng.standard_normal((64, 2, 64)) * 2.0, "bf16")
    Kf = bf16_to_f64(K)
    lo, hi = Kf.min(axis=0), Kf.max(axis=0)
    z = lo.astype(np.float32)
    s = ((hi - lo) / 3).astype(np.float32)
    codes = qk.quantize_k2(K, s, z, "bf16")
    at_min = Kf == lo[None]
    at_max = Kf == hi[None]
    assert (codes[at_min] == 0).all() and (codes[at_max] == 3).all()
    kh = qk.dequantize_k2(codes, s, z)
    np.testing.assert_allclose(kh[at_max], np.broadcast_to(hi, Kf.shape)[at_max], rtol=1e-6)
    np.testing.assert_array_equal(kh[at_min], np.broadcast_to(lo, Kf.shape)[at_min])
    mid = wl.f64_to_storage(np.array([[[-1.0 + 1.5 * 0.5]]]), "bf16")      # z=-1, s=0.5: u = 1.5
    assert qk.quantize_k2(mid, np.full((1, 1), 0.5, np.float32), np.full((1, 1), -1.0, np.float32),
                          "bf16")[0, 0, 0] == 2
