"""fp64 oracle of the int8 per-channel key cache (quantised KV).

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library.

What it follows (cited by title and section):

* "大模型推理加速：从 KV Cache 到投机采样的工程实践" (ybb.press), "KV Cache量化":
  the cache is normally 16-bit and quantising it to INT8 saves memory; keys are
  quantised per channel rather than per token because their channels are
  unevenly scaled.
* "LLM 推理优化：KV Cache、PagedAttention 与量化" (blog.tanteng.space), §4.2:
  keys per channel (small error), values kept in 16-bit; the sketch computes a
  channel's scale from the maximum magnitude over the token axis and stores
  round(k / scale) clamped to the signed range.

Readings (where the pages leave a step open):

* Symmetric int8 per channel: scale_c = amax_c / 127, code = clamp(rint(k /
  scale_c), -127, 127), k_hat = code * scale_c.  The printed sketch divides the
  amax by 2^bits - 1 but clamps to the signed range, which would clip every
  value above half the channel's amax; the symmetric form is the one whose
  clamp never triggers inside the calibration range.
* The scales are static per (KV head, channel) for a whole pool (calibrated on
  keys the caller has seen, as per-channel key quantisation with calibrated
  ranges does); a cache that is appended one token at a time cannot regroup
  earlier tokens.  Values outside the calibrated range clamp.
* The quotient k / scale is taken in float32 (IEEE division, round to nearest)
  and rounded half to even: the library decides the integer in the same
  precision.
* Values stay in the pool's 16-bit type; q and out share it.

Layout: the int8 K pool is [num_blocks][H_kv][d / 16][bs][16] -- the same
chunk-major tile order as the 16-bit K pool with 16 elements per 16-byte
chunk -- and the scales are float32 [H_kv][d].
"""
from __future__ import annotations

import numpy as np

from .paged_attention import (BLOCK_SIZE, _gqa_kv_head, attend_range, draft_limit, k_rows,
                              v_rows, widen)

K8_MAX = 127


def quantize_k(k: np.ndarray, k_scale: np.ndarray, dtype: str) -> np.ndarray:
    """Stored 16-bit key rows [..., H_kv, d] -> int8 codes of the same shape."""
    kf = widen(k, dtype).astype(np.float32)             # exact: 16-bit values fit float32
    quotient = kf / np.asarray(k_scale, dtype=np.float32)   # float32 division
    return np.clip(np.rint(quotient), -K8_MAX, K8_MAX).astype(np.int8)


def dequantize_k(codes: np.ndarray, k_scale: np.ndarray) -> np.ndarray:
    """int8 codes [..., H_kv, d] -> float64 code * scale (exact)."""
    return codes.astype(np.float64) * np.asarray(k_scale, dtype=np.float32).astype(np.float64)


def k8_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = BLOCK_SIZE):
    return (num_blocks, num_kv_heads, head_dim // 16, block_size, 16)


def write_kv_k8(k8_pool, v_pool, k_scale, k_new, v_new, slot_mapping, dtype):
    """Copies of the pools with token i's quantised K row and its V row stored at
    slot_mapping[i] (negative slots skipped).  k_new and v_new are [T][H_kv][d]
    in the 16-bit dtype."""
    k_out, v_out = k8_pool.copy(), v_pool.copy()
    codes = quantize_k(k_new, k_scale, dtype)
    n_kv, d = k_new.shape[1], k_new.shape[2]
    bs = k8_pool.shape[3]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = divmod(int(slot), bs)
        for g in range(n_kv):
            for c in range(d):
                k_out[b, g, c // 16, o, c % 16] = codes[i, g, c]
                v_out[b, g, c, o] = v_new[i, g, c]
    return k_out, v_out


def paged_decode_k8(q, k8_pool, v_pool, block_tables, context_lens, scale, k_scale, dtype):
    """Attention over the dequantised keys and the 16-bit values.

    q is [B][T][H_q][d] (T query tokens per sequence, the last T of the context,
    causal as in ``paged_verify``; T = 1 is decode).  Returns float64
    [B][T][H_q][d]."""
    B, T, Hq, d = q.shape
    Hkv = v_pool.shape[1]
    scale64 = float(np.float32(scale))
    out = np.zeros((B, T, Hq, d))
    for s in range(B):
        L = int(context_lens[s])
        for g in range(Hkv):
            K = dequantize_k(k_rows(k8_pool, block_tables[s], L, g), k_scale[g])
            V = widen(v_rows(v_pool, block_tables[s], L, g), dtype)
            for i in range(T):
                lim = draft_limit(L, T, i)
                for h in range(Hq):
                    if _gqa_kv_head(h, Hq, Hkv) == g:
                        out[s, i, h], _ = attend_range(widen(q[s, i, h], dtype), K[:lim], V[:lim],
                                                       scale64)
    return out


def paged_decode_k8_partials(q, k8_pool, v_pool, block_tables, context_lens, scale, k_scale,
                             dtype, partition_size: int, max_context_len: int):
    """Partition partials of ``paged_decode_k8``, rows ordered (s, i, h):
    o_part [B][T * H_q][n_parts][d], lse_part [B][T * H_q][n_parts]."""
    B, T, Hq, d = q.shape
    Hkv = v_pool.shape[1]
    P = max(1, -(-max_context_len // partition_size))
    scale64 = float(np.float32(scale))
    o_part = np.zeros((B, T * Hq, P, d))
    lse_part = np.full((B, T * Hq, P), -np.inf)
    for s in range(B):
        L = int(context_lens[s])
        for g in range(Hkv):
            K = dequantize_k(k_rows(k8_pool, block_tables[s], L, g), k_scale[g])
            V = widen(v_rows(v_pool, block_tables[s], L, g), dtype)
            for i in range(T):
                lim = draft_limit(L, T, i)
                for h in range(g * (Hq // Hkv), (g + 1) * (Hq // Hkv)):
                    qv = widen(q[s, i, h], dtype)
                    for p in range(P):
                        lo, hi = p * partition_size, min(lim, (p + 1) * partition_size)
                        if lo < hi:
                            o_part[s, i * Hq + h, p], lse_part[s, i * Hq + h, p] = attend_range(
                                qv, K[lo:hi], V[lo:hi], scale64)
    return o_part, lse_part
