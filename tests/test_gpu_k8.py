"""GPU parity of the int8-key cache (PA_K8_F16 / PA_K8_BF16) through the C ABI:
quantised append bit for bit against ``oracle.quantized_kv``, decode and verify
against the fp64 attention over the dequantised keys (tolerance 2e-2, the
16-bit value type's), block moves on pools whose K and V blocks differ in
size, and the 70B-style batch with per-channel key outliers at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import quantized_kv as qk
from paged_kv_cache_365_amd import pa
from paged_kv_cache_365_amd import workloads as wl
from paged_kv_cache_365_amd.device import to_numpy, to_torch, upload, widen_f32

from parity_bounds import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2
# A partition's log-sum-exp: the weights are rounded to the value type (2^-8
# for bf16, 2^-11 for f16), and the logits carry the rounding of q * scale to
# f16 for the matrix cores: |d logit| <= attention scale * 2^-11 * sum_c
# |q_c s_c code_c|, bounded per row over its tokens (lse moves by at most the
# largest logit error).
WEIGHT_U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def lse_bound(q, codes, scale, w, dtype):
    """Per-row bound [B][T * H_q] on the partial lse error (see above)."""
    from oracle.paged_attention import k_rows, widen
    B, T, Hq, d = q.shape
    G = Hq // w.num_kv_heads
    out = np.zeros((B, T * Hq))
    for s in range(B):
        L = int(w.context_lens[s])
        for g in range(w.num_kv_heads):
            kabs = np.abs(k_rows(codes, w.block_tables[s], L, g).astype(np.float64) * scale[g])
            for i in range(T):
                for h in range(g * G, (g + 1) * G):
                    qa = np.abs(widen(q[s, i, h], dtype))
                    worst = (kabs @ qa).max(initial=0.0)
                    out[s, i * Hq + h] = w.scale * 2.0 ** -11 * worst
    return out + WEIGHT_U[dtype] + 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pa.load()


def k8_tensor(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)


def f32_tensor(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


@pytest.mark.parametrize("dtype,d,hkv", [("bf16", 128, 8), ("f16", 64, 2), ("bf16", 64, 1)])
def test_write_kv_k8_bit_exact(dtype, d, hkv):
    rng = np.random.default_rng(21)
    nb, T = 9, 41
    scale = rng.uniform(0.005, 0.05, size=(hkv, d)).astype(np.float32)
    kp = np.full(qk.k8_pool_shape(nb, hkv, d), -128, np.int8)
    vp = wl.normal(rng, (nb, hkv, d, 16), dtype)
    # keys spanning past the calibrated range (clamped codes) and exact halves
    kn = wl.normal(rng, (T, hkv, d), dtype, gain=2.0)
    half = wl.f64_to_storage((np.arange(d) % 7 - 3 + 0.5) * scale[0].astype(np.float64), dtype)
    kn[0, 0] = half
    vn = wl.normal(rng, (T, hkv, d), dtype)
    slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int64)
    slots[[2, 30]] = -1
    want_k, want_v = qk.write_kv_k8(kp, vp, scale, kn, vn, slots, dtype)
    tk, tv = k8_tensor(kp), to_torch(vp, dtype, DEV)
    pa.pa_write_kv_k8(tk, tv, f32_tensor(scale), to_torch(kn, dtype, DEV), to_torch(vn, dtype, DEV),
                      torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(tk.cpu().numpy(), want_k)
    assert np.array_equal(to_numpy(tv).view(np.uint8), want_v.view(np.uint8))


CASES = [
    # V dtype, d, Hq, Hkv, T, partition
    ("bf16", 128, 64, 8, 1, 0), ("bf16", 128, 64, 8, 4, 0), ("bf16", 128, 16, 2, 1, 32),
    ("f16", 128, 32, 32, 1, 0), ("f16", 64, 8, 2, 3, 16), ("bf16", 64, 4, 4, 1, 0),
    ("f16", 128, 64, 8, 8, 48), ("bf16", 128, 64, 1, 1, 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_k8_random_cases(case):
    dtype, d, hq, hkv, T, P = CASES[case]
    lens = [1, T, 15, 16, 17, 64, 150, 300]
    w = wl.make_random_case(700 + case, num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                            head_dim=d, dtype=dtype, lens=lens)
    codes, scale = wl.k8_inputs(w, 710 + case, outlier_columns=max(1, hkv * d // 100))
    q = wl.normal(np.random.default_rng(720 + case), (len(lens), T, hq, d), dtype)
    dw = upload(w, DEV)
    tq = to_torch(q, dtype, DEV)
    ws = None
    if P:
        n = pa.pa_decode_workspace_bytes(len(lens), T * hq, d, w.max_context_len, P)
        ws = torch.empty(n // 4, dtype=torch.float32, device=DEV)
    out = pa.k8_attention(tq, k8_tensor(codes), dw.v_pool, f32_tensor(scale), dw.block_tables,
                          dw.context_lens, w.max_context_len, w.scale, partition_size=P, workspace=ws)
    torch.cuda.synchronize()
    got = widen_f32(out)
    want = qk.paged_decode_k8(q, codes, w.v_pool, w.block_tables, w.context_lens, w.scale, scale,
                              dtype)
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= TOL, f"{CASES[case]}: max-abs {err:.3e}"
    if P:
        n_parts = oracle.num_partitions(w.max_context_len, P)
        rows = len(lens) * T * hq
        wsn = ws.cpu().numpy()
        o_p = wsn[: rows * n_parts * d].reshape(len(lens), T * hq, n_parts, d).astype(np.float64)
        lse_p = wsn[rows * n_parts * d: rows * n_parts * (d + 1)].reshape(len(lens), T * hq, n_parts)
        wo, wlse = qk.paged_decode_k8_partials(q, codes, w.v_pool, w.block_tables, w.context_lens,
                                               w.scale, scale, dtype, P, w.max_context_len)
        live = np.isfinite(wlse)
        assert np.array_equal(np.isfinite(lse_p), live)
        bound = np.broadcast_to(lse_bound(q, codes, scale, w, dtype)[:, :, None], wlse.shape)
        assert (np.abs(lse_p[live] - wlse[live]) <= bound[live]).all()
        assert np.abs(o_p[live] - wo[live]).max(initial=0) <= TOL


def test_decode_k8_tiny_and_huge_scales():
    """The q operand is renormalised per row by a power of two, so key scales far
    from 1 keep full f16 precision."""
    dtype, d, hq, hkv = "bf16", 128, 16, 2
    lens = [33, 100]
    w = wl.make_random_case(731, num_seqs=2, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                            dtype=dtype, lens=lens)
    codes, scale = wl.k8_inputs(w, 732)
    q = wl.normal(np.random.default_rng(733), (2, 1, hq, d), dtype)
    dw = upload(w, DEV)
    for factor in (2.0 ** -12, 2.0 ** 10):
        sc = (scale * np.float32(factor)).astype(np.float32)
        out = pa.k8_attention(to_torch(q, dtype, DEV), k8_tensor(codes), dw.v_pool, f32_tensor(sc),
                              dw.block_tables, dw.context_lens, w.max_context_len,
                              float(np.float32(w.scale / factor)))
        torch.cuda.synchronize()
        want = qk.paged_decode_k8(q, codes, w.v_pool, w.block_tables, w.context_lens,
                                  float(np.float32(w.scale / factor)), sc, dtype)
        assert np.abs(widen_f32(out) - want).max() <= TOL, factor


@pytest.mark.parametrize("dtype,sign,P", [("f16", 1.0, 0), ("f16", -1.0, 64), ("bf16", 1.0, 64)])
def test_decode_k8_same_sign_query(dtype, sign, P):
    """Every query element of one sign: the sum Q of a row's operands -- and
    with it the code bias 144 Q the kernel removes once per row -- is as large
    as it gets, so the float32 cancellation is at its worst.  Outputs within
    the gates widened by the f16 query rounding, partial lse within its bound."""
    from parity_bounds import quantised_gates
    d, hq, hkv = 128, 16, 2
    lens = [1, 17, 300, 1000]
    w = wl.make_random_case(741, num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                            head_dim=d, dtype=dtype, lens=lens)
    codes, scale = wl.k8_inputs(w, 742, outlier_columns=2)
    rng = np.random.default_rng(743)
    q = wl.f64_to_storage(sign * (np.abs(rng.standard_normal((len(lens), 1, hq, d))) + 0.5), dtype)
    dw = upload(w, DEV)
    ws = None
    if P:
        n = pa.pa_decode_workspace_bytes(len(lens), hq, d, w.max_context_len, P)
        ws = torch.empty(n // 4, dtype=torch.float32, device=DEV)
    out = pa.k8_attention(to_torch(q, dtype, DEV), k8_tensor(codes), dw.v_pool, f32_tensor(scale),
                          dw.block_tables, dw.context_lens, w.max_context_len, w.scale,
                          partition_size=P, workspace=ws)
    torch.cuda.synchronize()
    want = qk.paged_decode_k8(q, codes, w.v_pool, w.block_tables, w.context_lens, w.scale, scale,
                              dtype)
    bound = lse_bound(q, codes, scale, w, dtype)
    qmag = float((bound - WEIGHT_U[dtype] - 1e-4).max()) * 2.0 ** 11
    v = oracle.widen(w.v_pool, dtype)
    gates = quantised_gates(dtype, qmag, float(np.abs(v[np.isfinite(v)]).max()))
    assert_parity(widen_f32(out), want, dtype, f"int8 keys, same-sign query {dtype} P{P}", **gates)
    if P:
        n_parts = oracle.num_partitions(w.max_context_len, P)
        rows = len(lens) * hq
        lse_p = ws.cpu().numpy()[rows * n_parts * d: rows * n_parts * (d + 1)].reshape(
            len(lens), hq, n_parts)
        _, wlse = qk.paged_decode_k8_partials(q, codes, w.v_pool, w.block_tables, w.context_lens,
                                              w.scale, scale, dtype, P, w.max_context_len)
        live = np.isfinite(wlse)
        assert np.array_equal(np.isfinite(lse_p), live)
        b = np.broadcast_to(bound[:, :, None], wlse.shape)
        assert (np.abs(lse_p[live] - wlse[live]) <= b[live]).all()


def test_block_moves_and_init_on_k8_pools():
    rng = np.random.default_rng(40)
    nb, hkv, d = 12, 4, 128
    codes = rng.integers(-127, 128, size=qk.k8_pool_shape(nb, hkv, d)).astype(np.int8)
    vp = wl.normal(rng, (nb, hkv, d, 16), "bf16")
    tk, tv = k8_tensor(codes), to_torch(vp, "bf16", DEV)
    pairs = np.array([[1, 9], [4, 10], [3, 3], [-1, 2]], np.int32)
    pa.pa_copy_blocks(tk, tv, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    want_k, want_v = oracle.copy_blocks(codes, vp, pairs)
    assert np.array_equal(tk.cpu().numpy(), want_k)
    assert np.array_equal(to_numpy(tv), want_v)
    ids = np.array([9, 0, 5], np.int32)
    gk = torch.zeros((3,) + codes.shape[1:], dtype=torch.int8, device=DEV)
    gv = torch.zeros((3,) + vp.shape[1:], dtype=torch.bfloat16, device=DEV)
    pa.pa_gather_blocks(tk, tv, torch.from_numpy(ids).to(DEV), gk, gv)
    torch.cuda.synchronize()
    assert np.array_equal(gk.cpu().numpy(), want_k[ids])
    assert np.array_equal(to_numpy(gv), want_v[ids])
    pa.pa_init_pool(tk, tv, 1)
    torch.cuda.synchronize()
    assert (tk.cpu().numpy() == -128).all() and torch.isnan(tv).all()


def test_k8_70b_gqa_4k_full():
    """The 70B-style batch (64 x 4096 tokens, 64/8 heads) with int8 keys carrying
    ten x10 outlier channels and bf16 values, unsplit as the benchmark runs it;
    every (sequence, head) row against the oracle, under both parity gates."""
    w = wl.make_config(2)
    codes, scale = wl.k8_inputs(w, 2042, outlier_columns=10)
    dw = upload(w, DEV)
    q = w.q[:, None]
    out = pa.k8_attention(to_torch(q, w.dtype, DEV), k8_tensor(codes), dw.v_pool, f32_tensor(scale),
                          dw.block_tables, dw.context_lens, w.max_context_len, w.scale)
    torch.cuda.synchronize()
    got = widen_f32(out)
    want = qk.paged_decode_k8(q, codes, w.v_pool, w.block_tables, w.context_lens, w.scale, scale,
                              w.dtype)
    assert_parity(got, want, w.dtype, "70b-gqa8-bf16-4k int8 keys (all rows)")