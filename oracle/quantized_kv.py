"""fp64 oracle of the quantised key caches: int8 keys with per-channel scales,
and 2-bit keys with a per-channel scale and zero point (KIVI).

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

The 2-bit key cache, its readings and its tile layout are described at its
section below.

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


def _decode_over_keys(q, keys, v_pool, block_tables, context_lens, scale, dtype):
    """Attention of q [B][T][H_q][d] (T query tokens per sequence, the last T of
    the context, causal as in ``paged_verify``; T = 1 is decode) over the float64
    key rows ``keys(s, g, L)`` [L][d] and the 16-bit V rows of the pool.  Returns
    float64 [B][T][H_q][d]."""
    B, T, Hq, d = q.shape
    Hkv = v_pool.shape[1]
    scale64 = float(np.float32(scale))
    out = np.zeros((B, T, Hq, d))
    for s in range(B):
        L = int(context_lens[s])
        for g in range(Hkv):
            K = keys(s, g, L)
            V = widen(v_rows(v_pool, block_tables[s], L, g), dtype)
            for i in range(T):
                lim = draft_limit(L, T, i)
                for h in range(Hq):
                    if _gqa_kv_head(h, Hq, Hkv) == g:
                        out[s, i, h], _ = attend_range(widen(q[s, i, h], dtype), K[:lim], V[:lim],
                                                       scale64)
    return out


def _partials_over_keys(q, keys, v_pool, block_tables, context_lens, scale, dtype,
                        partition_size: int, max_context_len: int):
    """Partition partials of ``_decode_over_keys``, rows ordered (s, i, h):
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
            K = keys(s, g, L)
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


def paged_decode_k8(q, k8_pool, v_pool, block_tables, context_lens, scale, k_scale, dtype):
    """Attention over the dequantised int8 keys and the 16-bit values; q is
    [B][T][H_q][d] (T = 1 is decode).  Returns float64 [B][T][H_q][d]."""
    keys = lambda s, g, L: dequantize_k(k_rows(k8_pool, block_tables[s], L, g), k_scale[g])
    return _decode_over_keys(q, keys, v_pool, block_tables, context_lens, scale, dtype)


def paged_decode_k8_partials(q, k8_pool, v_pool, block_tables, context_lens, scale, k_scale,
                             dtype, partition_size: int, max_context_len: int):
    """Partition partials of ``paged_decode_k8``, rows ordered (s, i, h):
    o_part [B][T * H_q][n_parts][d], lse_part [B][T * H_q][n_parts]."""
    keys = lambda s, g, L: dequantize_k(k_rows(k8_pool, block_tables[s], L, g), k_scale[g])
    return _partials_over_keys(q, keys, v_pool, block_tables, context_lens, scale, dtype,
                               partition_size, max_context_len)


# --------------------------------------------------------------------------
# 2-bit keys, asymmetric per channel (KIVI)
# --------------------------------------------------------------------------
# What it follows: §4.2 of the blog.tanteng.space page (KIVI): keys go to 2 bits
# per channel (the channel axis is where their error is small), values stay in
# 16 bits; its sketch computes a per-channel scale and zero point from the range
# over the token axis divided by 2^bits - 1.  "KV Cache量化" of the ybb.press
# page: KIVI quantises asymmetrically.
#
# Readings:
#
# * Asymmetric per channel: zero point z_c (the channel's calibrated minimum)
#   and step s_c = (max_c - min_c) / 3, codes 0..3, k_hat = z_c + s_c * code.
#   The sketch's divisor 2^bits - 1 is the asymmetric one (three steps span the
#   range); its signed clamp belongs to the symmetric form and is not taken.
# * As for int8 keys, z and s are static float32 per (KV head, channel) for the
#   pool, supplied by the caller; values outside [z, z + 3 s] clamp.
# * The code is decided in float32: u = (k - z) / s (IEEE subtraction and
#   division, round to nearest), code = rint(min(max(u, 0), 3)) with ties to
#   even, where max/min ignore a NaN (so 0/0, a constant channel at its zero
#   point, gives code 0; s = 0 with k above z gives 3, below z gives 0).
#
# Layout of a 2-bit key tile (bs tokens, d channels, bs * d / 16 words): uint32
# [4][bs][d / 64].  Channel c of the token at offset o lives in word
# [(c % 32) // 8][o][c // 64] at bit 2 * (4 * ((c // 32) % 2) + (c % 8) // 2)
# + 16 * (c % 2).  Each word holds 16 channels of one token.
K2_STEPS = 3        # 2^2 - 1 steps between the lowest and the highest code


def quantize_k2(k: np.ndarray, k_scale: np.ndarray, k_zero: np.ndarray, dtype: str) -> np.ndarray:
    """Stored 16-bit key rows [..., H_kv, d] -> 2-bit codes (uint8 0..3), same shape."""
    kf = widen(k, dtype).astype(np.float32)                     # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (kf - np.asarray(k_zero, np.float32)) / np.asarray(k_scale, np.float32)  # float32
    u = np.fmin(np.fmax(u, np.float32(0)), np.float32(K2_STEPS))  # fmax/fmin drop a NaN
    return np.rint(u).astype(np.uint8)


def dequantize_k2(codes: np.ndarray, k_scale: np.ndarray, k_zero: np.ndarray) -> np.ndarray:
    """2-bit codes [..., H_kv, d] -> float64 z + s * code."""
    s = np.asarray(k_scale, np.float32).astype(np.float64)
    z = np.asarray(k_zero, np.float32).astype(np.float64)
    return z + s * codes.astype(np.float64)


def k2_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = BLOCK_SIZE):
    return (num_blocks, num_kv_heads, 4, block_size, head_dim // 64)


def k2_position(c: int):
    """(word index [group][.][col], bit) of channel c inside a token's words."""
    return (c % 32) // 8, c // 64, 2 * (4 * ((c // 32) % 2) + (c % 8) // 2) + 16 * (c % 2)


def k2_rows(k2_pool: np.ndarray, table_row: np.ndarray, length: int, kv_head: int) -> np.ndarray:
    """2-bit codes [length][d] of one KV head of one sequence, in token order."""
    bs = k2_pool.shape[3]
    d = 64 * k2_pool.shape[4]
    t = np.arange(length)
    physical = table_row[t // bs]
    offset = t % bs
    rows = np.empty((length, d), np.uint8)
    for c in range(d):
        grp, col, bit = k2_position(c)
        words = k2_pool[physical, kv_head, grp, offset, col].astype(np.uint64)
        rows[:, c] = (words >> np.uint64(bit)) & np.uint64(3)
    return rows


def write_kv_k2(k2_pool, v_pool, k_scale, k_zero, k_new, v_new, slot_mapping, dtype):
    """Copies of the pools with token i's 2-bit key row and its V row stored at
    slot_mapping[i] (negative slots skipped).  A written token's key words are
    replaced whole."""
    k_out, v_out = k2_pool.copy(), v_pool.copy()
    codes = quantize_k2(k_new, k_scale, k_zero, dtype)
    n_kv, d = k_new.shape[1], k_new.shape[2]
    bs = k2_pool.shape[3]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = divmod(int(slot), bs)
        for g in range(n_kv):
            words = np.zeros((4, d // 64), np.uint64)
            for c in range(d):
                grp, col, bit = k2_position(c)
                words[grp, col] |= np.uint64(int(codes[i, g, c]) << bit)
            k_out[b, g, :, o, :] = words.astype(np.uint32)
            v_out[b, g, :, o] = v_new[i, g, :]
    return k_out, v_out


def paged_decode_k2(q, k2_pool, v_pool, block_tables, context_lens, scale, k_scale, k_zero, dtype):
    """Attention over the dequantised 2-bit keys and the 16-bit values; q is
    [B][T][H_q][d] (T = 1 is decode).  Returns float64 [B][T][H_q][d]."""
    keys = lambda s, g, L: dequantize_k2(k2_rows(k2_pool, block_tables[s], L, g), k_scale[g],
                                         k_zero[g])
    return _decode_over_keys(q, keys, v_pool, block_tables, context_lens, scale, dtype)


def paged_decode_k2_partials(q, k2_pool, v_pool, block_tables, context_lens, scale, k_scale,
                             k_zero, dtype, partition_size: int, max_context_len: int):
    """Partition partials of ``paged_decode_k2``, rows ordered (s, i, h)."""
    keys = lambda s, g, L: dequantize_k2(k2_rows(k2_pool, block_tables[s], L, g), k_scale[g],
                                         k_zero[g])
    return _partials_over_keys(q, keys, v_pool, block_tables, context_lens, scale, dtype,
                               partition_size, max_context_len)
