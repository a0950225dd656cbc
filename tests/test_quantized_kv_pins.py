"""Pins for the int8 per-channel key oracle (``oracle/quantized_kv.py``):
exact codes for exactly representable quotients, rounding and clamping rules,
the per-channel error bound, a dense brute force over the dequantised keys
written here, the KV append, and the property the pages give for per-channel
key quantisation (keys with a few outlier channels lose far less than with one
scale for the whole tensor: "KV Cache量化" of the ybb.press page, §4.2 of the
blog.tanteng.space page).
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import quantized_kv as qk
from paged_kv_cache_365_amd import workloads as wl

BS = 16


def f16(a):
    return np.asarray(a, dtype=np.float16)


def test_codes_of_exact_quotients_round_and_clamp():
    s = np.float32(2.0 ** -5)
    scale = np.full((1, 4), s, np.float32)
    n = np.arange(-100, 101)
    cases = {0.0: n, 0.4: n, 0.6: n + 1, -0.4: n, -0.6: n - 1}
    for frac, want in cases.items():
        k = f16((n + frac) * float(s))[:, None, None] * np.ones((1, 1, 4), np.float16)
        got = qk.quantize_k(k, scale, "f16")[:, 0, 0]
        assert np.array_equal(got, want), frac
    # exact halves go to the even code
    k = f16((n + 0.5) * float(s))[:, None, None] * np.ones((1, 1, 4), np.float16)
    got = qk.quantize_k(k, scale, "f16")[:, 0, 0]
    assert np.array_equal(got, np.where((n % 2) == 0, n, n + 1))
    # out of range clamps to +-127 (never -128)
    k = f16(np.array([200, -200, 127.4, -127.6, 1e4]) * float(s))[:, None, None] * np.ones((1, 1, 4), np.float16)
    assert qk.quantize_k(k, scale, "f16")[:, 0, 0].tolist() == [127, -127, 127, -127, 127]


def test_each_channel_uses_its_own_scale():
    rng = np.random.default_rng(1)
    Hkv, d = 2, 64
    scale = (2.0 ** -rng.integers(2, 9, size=(Hkv, d))).astype(np.float32)
    n = rng.integers(-120, 121, size=(5, Hkv, d))
    k = wl.f64_to_storage(n * scale.astype(np.float64), "bf16")   # n * 2^-e: exact in bf16 for |n| < 256
    assert np.array_equal(qk.quantize_k(k, scale, "bf16"), n.astype(np.int8))
    assert np.array_equal(qk.dequantize_k(n.astype(np.int8), scale), n * scale.astype(np.float64))


def test_error_bound_half_a_step():
    rng = np.random.default_rng(2)
    Hkv, d = 2, 128
    scale = rng.uniform(0.01, 0.2, size=(Hkv, d)).astype(np.float32)
    k = wl.f64_to_storage(rng.uniform(-126.9, 126.9, size=(50, Hkv, d)) * scale, "f16")
    kf = k.astype(np.float64)
    err = np.abs(qk.dequantize_k(qk.quantize_k(k, scale, "f16"), scale) - kf)
    assert (err <= scale.astype(np.float64) * (0.5 + 2.0 ** -16)).all()


def pack_k8(codes, lens, rng, extra_blocks=2):
    """Contiguous codes [B][L][H_kv][d] -> a permuted int8 pool and tables, with
    this test's own index arithmetic (16 channels per 16-byte chunk)."""
    B, Lmax, Hkv, d = codes.shape
    need = [-(-int(L) // BS) for L in lens]
    nb = sum(need) + extra_blocks
    perm = rng.permutation(nb)
    tables = np.full((B, max(max(need), 1)), -1, np.int32)
    pool = np.full((nb, Hkv, d // 16, BS, 16), -128, np.int8)
    c = 0
    for s in range(B):
        for j in range(need[s]):
            tables[s, j] = perm[c]
            c += 1
        for t in range(int(lens[s])):
            b, o = tables[s, t // BS], t % BS
            for g in range(Hkv):
                for ch in range(d):
                    pool[b, g, ch // 16, o, ch % 16] = codes[s, t, g, ch]
    return pool, tables


def pack_v(V, tables, lens, nb):
    B, Lmax, Hkv, d = V.shape
    vp = wl.nan_fill((nb, Hkv, d, BS), "bf16")
    for s in range(B):
        for t in range(int(lens[s])):
            vp[tables[s, t // BS], :, :, t % BS] = V[s, t]
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


@pytest.mark.parametrize("T", [1, 3])
def test_decode_equals_dense_over_dequantised_keys(T):
    rng = np.random.default_rng(3 + T)
    B, Hkv, G, d = 3, 2, 4, 64
    lens = [T, 21, 50]
    Lmax = max(lens)
    codes = rng.integers(-127, 128, size=(B, Lmax, Hkv, d)).astype(np.int8)
    scale = rng.uniform(0.005, 0.05, size=(Hkv, d)).astype(np.float32)
    V = wl.normal(rng, (B, Lmax, Hkv, d), "bf16")
    q = wl.normal(rng, (B, T, Hkv * G, d), "bf16")
    pool, tables = pack_k8(codes, lens, rng)
    vp = pack_v(V, tables, lens, pool.shape[0])
    got = qk.paged_decode_k8(q, pool, vp, tables, np.array(lens, np.int32), 0.125, scale, "bf16")
    for s in range(B):
        L = lens[s]
        Kd = codes[s, :L].astype(np.float64) * scale.astype(np.float64)     # [L][H_kv][d]
        Vd = (V[s, :L].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        qd = (q[s].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        np.testing.assert_allclose(got[s], dense_causal(qd, Kd, Vd, 0.125), rtol=0, atol=1e-12)


def test_partials_merge_to_decode():
    from oracle import merge_partials
    rng = np.random.default_rng(9)
    B, Hkv, G, d, T = 2, 2, 2, 64, 2
    lens = [7, 40]
    codes = rng.integers(-127, 128, size=(B, 40, Hkv, d)).astype(np.int8)
    scale = rng.uniform(0.005, 0.05, size=(Hkv, d)).astype(np.float32)
    V = wl.normal(rng, (B, 40, Hkv, d), "f16")
    q = wl.normal(rng, (B, T, Hkv * G, d), "f16")
    pool, tables = pack_k8(codes, lens, rng)
    vp = np.zeros((pool.shape[0], Hkv, d, BS), np.float16)
    for s in range(B):
        for t in range(lens[s]):
            vp[tables[s, t // BS], :, :, t % BS] = V[s, t]
    want = qk.paged_decode_k8(q, pool, vp, tables, np.array(lens), 0.1, scale, "f16")
    o, lse = qk.paged_decode_k8_partials(q, pool, vp, tables, np.array(lens), 0.1, scale, "f16",
                                         16, 40)
    np.testing.assert_allclose(merge_partials(o, lse).reshape(want.shape), want, rtol=0, atol=1e-13)


def test_write_kv_k8_places_codes_and_values():
    rng = np.random.default_rng(4)
    nb, Hkv, d, T = 5, 2, 64, 12
    scale = rng.uniform(0.01, 0.05, size=(Hkv, d)).astype(np.float32)
    kp = np.full(qk.k8_pool_shape(nb, Hkv, d), -128, np.int8)
    vp = wl.normal(rng, (nb, Hkv, d, BS), "bf16")
    kn = wl.normal(rng, (T, Hkv, d), "bf16")
    vn = wl.normal(rng, (T, Hkv, d), "bf16")
    slots = rng.choice(nb * BS, size=T, replace=False).astype(np.int64)
    slots[4] = -1
    k2, v2 = qk.write_kv_k8(kp, vp, scale, kn, vn, slots, "bf16")
    codes = qk.quantize_k(kn, scale, "bf16")
    ke, ve = kp.copy(), vp.copy()
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        b, o = divmod(int(sl), BS)
        for g in range(Hkv):
            for ch in range(d):
                ke[b, g, ch // 16, o, ch % 16] = codes[i, g, ch]
                ve[b, g, ch, o] = vn[i, g, ch]
    assert np.array_equal(k2, ke) and np.array_equal(v2, ve)


def test_per_channel_scales_beat_one_scale_on_outlier_channels():
    """Keys whose few outlier channels are 10x the rest: per-channel int8 keeps the
    attention output close to the unquantised one; a single scale for the tensor
    spends its range on the outliers and loses far more."""
    rng = np.random.default_rng(5)
    L, Hkv, G, d = 512, 1, 8, 128
    K = rng.standard_normal((L, Hkv, d))
    K[:, 0, rng.choice(d, 2, replace=False)] *= 10.0
    Kb = wl.f64_to_storage(K, "bf16")
    Kf = (Kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    V = rng.standard_normal((L, Hkv, d))
    q = rng.standard_normal((1, Hkv * G, d))
    exact = dense_causal(q, Kf, V, d ** -0.5)
    amax_c = np.abs(Kf).max(axis=0)                        # [H_kv][d]
    per_channel = (amax_c / 127).astype(np.float32)
    per_tensor = np.full_like(per_channel, np.float32(np.abs(Kf).max() / 127))
    errs = {}
    for name, sc in [("channel", per_channel), ("tensor", per_tensor)]:
        Kq = qk.dequantize_k(qk.quantize_k(Kb, sc, "bf16"), sc)
        errs[name] = np.abs(dense_causal(q, Kq, V, d ** -0.5) - exact).max()
    assert errs["channel"] < 0.02
    assert errs["tensor"] > 3 * errs["channel"]
