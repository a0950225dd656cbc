"""GPU parity with 8-token blocks (the smaller block size §2.2 of the
blog.tanteng.space page mentions for 70B models) through the C ABI: gather
indices, KV append (16-bit and int8 keys) and block moves bit for bit, decode
and verify against the fp64 oracle, the same context stored in 8- and 16-token
blocks giving bit-identical outputs (the kernel steps 16 tokens at a time
either way), and the 70B-style batch at full size.
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
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pa.load()


def _bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


def test_slot_ids_8_token_blocks():
    tables = torch.tensor([[7, 2, 11, -1]], dtype=torch.int32, device=DEV)
    lens = torch.tensor([20], dtype=torch.int32, device=DEV)
    out = torch.empty((1, 24), dtype=torch.int64, device=DEV)
    pa.pa_debug_slot_ids(tables, lens, 24, 12, out, block_size=8)
    torch.cuda.synchronize()
    want = oracle.slot_ids(np.array([[7, 2, 11, -1]]), np.array([20]), 24, 8)
    assert np.array_equal(out.cpu().numpy(), want)
    w = wl.make_config(3, block_size=8)
    dw = upload(w, DEV)
    out = torch.empty((w.num_seqs, w.max_context_len), dtype=torch.int64, device=DEV)
    pa.pa_debug_slot_ids(dw.block_tables, dw.context_lens, w.max_context_len, w.num_blocks, out,
                         block_size=8)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(),
                          oracle.slot_ids(w.block_tables, w.context_lens, w.max_context_len, 8))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_write_kv_8_token_blocks(dtype, d):
    rng = np.random.default_rng(31)
    nb, hkv, T = 10, 2, 33
    ks, vs = wl.pool_shapes(nb, hkv, d, dtype, 8)
    kp, vp = wl.normal(rng, ks, dtype), wl.normal(rng, vs, dtype)
    kn, vn = wl.normal(rng, (T, hkv, d), dtype), wl.normal(rng, (T, hkv, d), dtype)
    slots = rng.choice(nb * 8, size=T, replace=False).astype(np.int64)
    slots[3] = -1
    want_k, want_v = oracle.write_kv(kp, vp, kn, vn, slots)
    tk, tv = to_torch(kp, dtype, DEV), to_torch(vp, dtype, DEV)
    pa.pa_write_kv(tk, tv, to_torch(kn, dtype, DEV), to_torch(vn, dtype, DEV),
                   torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(to_numpy(tk)), _bytes(want_k))
    assert np.array_equal(_bytes(to_numpy(tv)), _bytes(want_v))


def test_write_kv_k8_and_block_moves_8_token_blocks():
    rng = np.random.default_rng(32)
    nb, hkv, d, T = 12, 2, 128, 40
    scale = rng.uniform(0.01, 0.05, size=(hkv, d)).astype(np.float32)
    kp = np.full(qk.k8_pool_shape(nb, hkv, d, 8), -128, np.int8)
    vp = wl.normal(rng, (nb, hkv, d, 8), "bf16")
    kn, vn = wl.normal(rng, (T, hkv, d), "bf16"), wl.normal(rng, (T, hkv, d), "bf16")
    slots = rng.choice(nb * 8, size=T, replace=False).astype(np.int64)
    want_k, want_v = qk.write_kv_k8(kp, vp, scale, kn, vn, slots, "bf16")
    tk, tv = torch.from_numpy(kp).to(DEV), to_torch(vp, "bf16", DEV)
    pa.pa_write_kv_k8(tk, tv, torch.from_numpy(scale).to(DEV), to_torch(kn, "bf16", DEV),
                      to_torch(vn, "bf16", DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(tk.cpu().numpy(), want_k)
    assert np.array_equal(_bytes(to_numpy(tv)), _bytes(want_v))
    pairs = np.array([[1, 9], [4, 10], [2, 2]], np.int32)
    pa.pa_copy_blocks(tk, tv, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    ck, cv = oracle.copy_blocks(want_k, want_v, pairs)
    assert np.array_equal(tk.cpu().numpy(), ck)
    assert np.array_equal(_bytes(to_numpy(tv)), _bytes(cv))


CASES = [
    # dtype, d, Hq, Hkv, T, partition, int8 keys
    ("bf16", 128, 64, 8, 1, 0, False), ("bf16", 128, 64, 8, 4, 0, False),
    ("f16", 128, 32, 32, 1, 32, False), ("f32", 64, 8, 2, 1, 0, False),
    ("bf16", 64, 16, 2, 3, 16, False), ("bf16", 128, 64, 8, 1, 0, True),
    ("f16", 128, 16, 2, 2, 48, True), ("f32", 128, 8, 4, 2, 16, False),
    ("bf16", 128, 64, 8, 8, 0, False), ("f16", 64, 32, 4, 5, 32, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_8_token_blocks(case):
    dtype, d, hq, hkv, T, P, k8 = CASES[case]
    lens = [1, 7, 8, 9, 15, 16, 17, 23, 63, 150, 301]
    w = wl.make_random_case(600 + case, num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv,
                            head_dim=d, dtype=dtype, lens=lens, block_size=8)
    dw = upload(w, DEV)
    q = wl.normal(np.random.default_rng(610 + case), (len(lens), T, hq, d), dtype)
    tq = to_torch(q, dtype, DEV)
    if k8:
        codes, scale = wl.k8_inputs(w, 620 + case)
        out = pa.k8_attention(tq, torch.from_numpy(codes).to(DEV), dw.v_pool,
                              torch.from_numpy(scale).to(DEV), dw.block_tables, dw.context_lens,
                              w.max_context_len, w.scale, partition_size=P)
        want = qk.paged_decode_k8(q, codes, w.v_pool, w.block_tables, w.context_lens, w.scale,
                                  scale, dtype)
    else:
        out = pa.verify_attention(tq, dw.k_pool, dw.v_pool, dw.block_tables, dw.context_lens,
                                  w.max_context_len, w.scale, partition_size=P)
        want = oracle.paged_verify(q, w.k_pool, w.v_pool, w.block_tables, w.context_lens,
                                   w.scale, dtype)
    torch.cuda.synchronize()
    got = widen_f32(out)
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= TOL[dtype], f"{CASES[case]}: max-abs {err:.3e}"


def pack(K, V, lens, bs, rng, dtype):
    """Contiguous K, V [B][L][H_kv][d] -> pools of bs-token blocks and tables,
    with this test's own index arithmetic."""
    B, Lmax, Hkv, d = K.shape
    need = [-(-L // bs) for L in lens]
    nb = sum(need) + 3
    perm = rng.permutation(nb)
    ks, vs = wl.pool_shapes(nb, Hkv, d, dtype, bs)
    kp = wl.nan_fill(ks, dtype)
    vp = wl.nan_fill(vs, dtype)
    x = ks[4]
    tables = np.full((B, max(need)), -1, np.int32)
    c = 0
    for s in range(B):
        tables[s, :need[s]] = perm[c:c + need[s]]
        c += need[s]
        for t in range(lens[s]):
            b, o = tables[s, t // bs], t % bs
            for ch in range(d):
                kp[b, :, ch // x, o, ch % x] = K[s, t, :, ch]
                vp[b, :, ch, o] = V[s, t, :, ch]
    return kp, vp, tables


@pytest.mark.parametrize("P", [0, 32])
def test_8_and_16_token_blocks_are_bit_identical(P):
    rng = np.random.default_rng(33)
    dtype, B, hkv, hq, d = "bf16", 4, 2, 16, 128
    lens = [5, 40, 77, 130]
    K = wl.normal(rng, (B, max(lens), hkv, d), dtype)
    V = wl.normal(rng, (B, max(lens), hkv, d), dtype)
    q = to_torch(wl.normal(rng, (B, hq, d), dtype), dtype, DEV)
    outs = []
    for bs in (16, 8):
        kp, vp, tab = pack(K, V, lens, bs, rng, dtype)
        out = pa.paged_attention(q, to_torch(kp, dtype, DEV), to_torch(vp, dtype, DEV),
                                 torch.from_numpy(tab).to(DEV),
                                 torch.tensor(lens, dtype=torch.int32, device=DEV), max(lens),
                                 float(np.float32(d ** -0.5)), partition_size=P)
        torch.cuda.synchronize()
        outs.append(to_numpy(out))
    assert np.array_equal(outs[0], outs[1])


def test_70b_gqa_4k_8_token_blocks_full():
    """The 70B-style batch cut into 8-token blocks: every row against the
    oracle, under both parity gates."""
    w = wl.make_config(2, block_size=8)
    dw = upload(w, DEV)
    out = pa.paged_attention(dw.q, dw.k_pool, dw.v_pool, dw.block_tables, dw.context_lens,
                             w.max_context_len, w.scale)
    torch.cuda.synchronize()
    want = oracle.paged_decode(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale,
                               w.dtype)
    assert_parity(widen_f32(out), want, w.dtype, "70b-gqa8-bf16-4k-bs8 (all rows)")
