"""fp64 CPU oracle for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (no kernels, headers, tables or helpers); both read their
inputs from the seeded generators alone.

It is the plain definition, written for a reader to check by eye, not the
method's fast form.  The pages it follows (cited by title and section):

* [P1] "LLM推理优化实战：从KV Cache到Speculative Decoding，把延迟打下来"
       (jsqmd.com), section "KV Cache：推理加速的第一板斧", the KVCacheAttention
       listing: scale is head_dim^-0.5, softmax runs over the key axis, and the
       new token's K/V is appended to the cache before attention is taken.
* [P2] "大模型推理加速：从 KV Cache 到投机采样的工程实践" (ybb.press), section
       "主流优化策略": MQA/GQA, query heads grouped onto shared KV heads.
* [P3] "LLM 推理优化：KV Cache、PagedAttention 与量化" (blog.tanteng.space),
       §2.2 (16-token blocks, block table from logical to physical blocks) and
       §2.3 (blocks shared between block tables for a common prefix).
* [P4] "大模型推理加速与显存黑科技 (Inference Acceleration & KV Cache)"
       (ialgorithm.me), §2 attention equation softmax(QK^T/sqrt(d_k))V;
       §3.2 block-table figure (block i holds tokens 16i..16i+15, logical
       blocks 0/1/2 map to physical #7/#2/#11); §4.2 online softmax is exact.

Readings taken where the pages are silent:

* GQA grouping is contiguous: q-head h reads KV head h // (H_q / H_kv).
* A context of length 0 attends to nothing: the output row is 0 and every
  partition partial is (0, -inf).
* ``scale`` is the float32 the caller passes; the oracle widens it exactly.
* Inputs are read from their stored bits and widened exactly to fp64.

Every function below is pinned in ``tests/test_oracle_pins.py`` against brute
force, closed forms and invariants that do not reuse this code.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16  # tokens per physical block [P3 §2.2; P4 §3.2]


# --------------------------------------------------------------------------
# exact widening of stored elements
# --------------------------------------------------------------------------
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored elements -> float64, exactly.

    f32 and f16 widen directly; bf16 is the upper half of an IEEE float32, so its
    16 stored bits are shifted into the high half of a 32-bit word and read as
    float32 before widening.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# block-table address arithmetic  [P3 §2.2; P4 §3.2 block-table figure]
# --------------------------------------------------------------------------
def slot_of(table_row: np.ndarray, t: int, block_size: int = BLOCK_SIZE) -> int:
    """Token t sits in logical block t // bs at offset t % bs (bs = 16 by default;
    the 8-token variant of [P3] §2.2 as well); the table maps the logical block to
    a physical one; the slot is physical * bs + offset."""
    logical = t // block_size
    offset = t % block_size
    physical = int(table_row[logical])
    return physical * block_size + offset


def slot_ids(block_tables: np.ndarray, context_lens: np.ndarray, max_context_len: int,
             block_size: int = BLOCK_SIZE) -> np.ndarray:
    """int64 [B][max_context_len]: the slot of every live token, -1 past the length."""
    B = len(context_lens)
    out = np.full((B, max_context_len), -1, dtype=np.int64)
    for s in range(B):
        for t in range(min(int(context_lens[s]), max_context_len)):
            out[s, t] = slot_of(block_tables[s], t, block_size)
    return out


def tile_byte_offset(physical: int, kv_head: int, num_kv_heads: int, head_dim: int,
                     elem_bytes: int, block_size: int = BLOCK_SIZE) -> int:
    """Byte offset of tile (physical block, kv head) in a pool of bs * d-element
    tiles ordered block-major, then by KV head."""
    tile_bytes = block_size * head_dim * elem_bytes
    return (physical * num_kv_heads + kv_head) * tile_bytes


# Pool layouts (the library's ABI; only the order of elements inside a tile
# differs between K and V; bs = tokens per block, read from the pool's shape):
#   K  [blocks][H_kv][d / x][bs][x]   x = elements per 16-byte chunk: element c
#                                      of the token at offset o is at [c // x][o][c % x]
#   V  [blocks][H_kv][d][bs]          element c of the token at offset o is at [c][o]
def k_rows(k_pool: np.ndarray, table_row: np.ndarray, length: int, kv_head: int) -> np.ndarray:
    """K rows [length][d] (stored dtype) of one KV head of one sequence, in token
    order: row t comes from physical block table_row[t // bs] at offset t % bs."""
    bs = k_pool.shape[3]
    t = np.arange(length)
    physical = table_row[t // bs]
    offset = t % bs
    n_chunks, x = k_pool.shape[2], k_pool.shape[4]
    rows = np.empty((length, n_chunks, x), dtype=k_pool.dtype)
    for c in range(n_chunks):
        rows[:, c, :] = k_pool[physical, kv_head, c, offset, :]
    return rows.reshape(length, n_chunks * x)


def v_rows(v_pool: np.ndarray, table_row: np.ndarray, length: int, kv_head: int) -> np.ndarray:
    """V rows [length][d] (stored dtype), in token order, from the [d][bs] tiles."""
    bs = v_pool.shape[3]
    t = np.arange(length)
    physical = table_row[t // bs]
    offset = t % bs
    d = v_pool.shape[2]
    rows = np.empty((length, d), dtype=v_pool.dtype)
    for c in range(d):
        rows[:, c] = v_pool[physical, kv_head, c, offset]
    return rows


# --------------------------------------------------------------------------
# attention of one query head over a contiguous token range
# --------------------------------------------------------------------------
def attend_range(q_vec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Two-pass softmax attention of one query over rows K, V (already fp64).

    Returns (out, lse) with lse = ln sum_t exp(x_t), x_t = scale * q.k_t
    [P4 §2 attention equation; P1 KVCacheAttention listing].  An empty range
    returns (0, -inf).
    """
    d = q_vec.shape[0]
    if K.shape[0] == 0:
        return np.zeros(d), -np.inf
    x = scale * (K @ q_vec)            # logits, one per token
    m = x.max()                        # subtract the max before exponentiating
    w = np.exp(x - m)
    z = w.sum()
    out = (w @ V) / z
    return out, m + np.log(z)


def _gqa_kv_head(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Contiguous query-head groups share one KV head [P2 "主流优化策略"]."""
    group = num_q_heads // num_kv_heads
    return h // group


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, scale, dtype,
                 pairs=None) -> np.ndarray:
    """out[s][h] = softmax(scale * q[s,h] K_s^T) V_s over the gathered context.

    ``q`` [B][H_q][d]; pools [NB][H_kv][16][d]; all in stored form.  ``pairs``
    optionally restricts the work to a list of (s, h); the other rows are NaN.
    Returns float64 [B][H_q][d].
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    scale64 = float(np.float32(scale))
    todo = pairs if pairs is not None else [(s, h) for s in range(B) for h in range(Hq)]
    out = np.full((B, Hq, d), np.nan) if pairs is not None else np.zeros((B, Hq, d))
    by_head = {}
    for s, h in todo:
        by_head.setdefault((s, _gqa_kv_head(h, Hq, Hkv)), []).append(h)
    for (s, g), heads in by_head.items():
        L = int(context_lens[s])
        K = widen(k_rows(k_pool, block_tables[s], L, g), dtype)
        V = widen(v_rows(v_pool, block_tables[s], L, g), dtype)
        for h in heads:
            out[s, h], _ = attend_range(widen(q[s, h], dtype), K, V, scale64)
    return out


def num_partitions(max_context_len: int, partition_size: int) -> int:
    return max(1, -(-max_context_len // partition_size))


def paged_decode_partials(q, k_pool, v_pool, block_tables, context_lens, scale, dtype,
                          partition_size: int, max_context_len: int | None = None):
    """Per partition p, the attention over tokens [pP, min(L, (p+1)P)).

    Returns (o_part [B][H_q][n_parts][d], lse_part [B][H_q][n_parts]) in float64;
    o_part is normalised within its partition and lse_part = ln sum exp(x_t) over
    it.  Empty partitions give (0, -inf).
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if max_context_len is None:
        max_context_len = int(np.max(context_lens)) if len(context_lens) else 0
    P = num_partitions(max_context_len, partition_size)
    scale64 = float(np.float32(scale))
    o_part = np.zeros((B, Hq, P, d))
    lse_part = np.full((B, Hq, P), -np.inf)
    for s in range(B):
        L = int(context_lens[s])
        for g in range(Hkv):
            K = widen(k_rows(k_pool, block_tables[s], L, g), dtype)
            V = widen(v_rows(v_pool, block_tables[s], L, g), dtype)
            for h in range(g * (Hq // Hkv), (g + 1) * (Hq // Hkv)):
                qv = widen(q[s, h], dtype)
                for p in range(P):
                    lo, hi = p * partition_size, min(L, (p + 1) * partition_size)
                    if lo >= hi:
                        continue
                    o_part[s, h, p], lse_part[s, h, p] = attend_range(qv, K[lo:hi], V[lo:hi], scale64)
    return o_part, lse_part


def merge_partials(o_part: np.ndarray, lse_part: np.ndarray) -> np.ndarray:
    """Log-sum-exp merge of partition results.

    With M = max_p lse_p and LSE = M + ln sum_p exp(lse_p - M), the full result
    is sum_p exp(lse_p - LSE) o_p: each partial is re-weighted by its share of
    the total softmax mass, which is why streaming the normaliser is exact
    [P4 §4.2].  Rows whose partials are all empty give 0.
    """
    B, Hq, P, d = o_part.shape
    out = np.zeros((B, Hq, d))
    for s in range(B):
        for h in range(Hq):
            lse = lse_part[s, h]
            M = lse.max()
            if not np.isfinite(M):
                continue
            total = M + np.log(np.exp(lse - M).sum())
            weights = np.exp(lse - total)
            out[s, h] = weights @ o_part[s, h]
    return out


# --------------------------------------------------------------------------
# KV append  [P1 KVCacheAttention listing: new K/V joins the cache first;
#             P3 §2.3: a block is taken from the pool when it is written]
# --------------------------------------------------------------------------
def write_kv(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Copies of the pools with token i's [H_kv][d] rows stored at slot_mapping[i].

    A slot is physical * bs + offset; negative slots are skipped.  Values are
    copied bit for bit into the K and V tile layouts described above.
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    n_kv, n_chunks, bs, x = k_pool.shape[1], k_pool.shape[2], k_pool.shape[3], k_pool.shape[4]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = divmod(int(slot), bs)
        for g in range(n_kv):
            for c in range(n_chunks * x):
                k_out[b, g, c // x, o, c % x] = k_new[i, g, c]
                v_out[b, g, c, o] = v_new[i, g, c]
    return k_out, v_out


# --------------------------------------------------------------------------
# whole-block moves  [P3 §2.3 (2): the copy of a copy-on-write;
#                     P3 §2.3 (1): swapping a preempted request's blocks out]
# --------------------------------------------------------------------------
def copy_blocks(k_pool, v_pool, pairs):
    """Copies of the pools in which block dst of each (src, dst) pair holds what
    block src held before the call (every KV head, K and V).  Pairs naming a
    block outside the pool, or with src == dst, are skipped."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    nb = k_pool.shape[0]
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < nb and 0 <= dst < nb) or src == dst:
            continue
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
    return k_out, v_out


def gather_blocks(k_pool, v_pool, block_ids, k_dst, v_dst):
    """Copies of the packed buffers (shaped [n] + one block's shape) in which
    entry i holds pool block block_ids[i]; ids outside the pool leave entry i as
    it was."""
    k_out, v_out = k_dst.copy(), v_dst.copy()
    for i, b in enumerate(np.asarray(block_ids, dtype=np.int64)):
        if 0 <= b < k_pool.shape[0]:
            k_out[i] = k_pool[b]
            v_out[i] = v_pool[b]
    return k_out, v_out


def scatter_blocks(k_pool, v_pool, block_ids, k_src, v_src):
    """Copies of the pools in which block block_ids[i] holds packed entry i; ids
    outside the pool are skipped."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    for i, b in enumerate(np.asarray(block_ids, dtype=np.int64)):
        if 0 <= b < k_pool.shape[0]:
            k_out[b] = k_src[i]
            v_out[b] = v_src[i]
    return k_out, v_out


# --------------------------------------------------------------------------
# speculative-decoding verify: T draft tokens per sequence in one call
# [P1 SpeculativeDecoder listing: the target model runs once over the context
#  followed by the draft tokens; P3 §6.2 and P4 §5.1: all candidates are
#  checked in one forward pass]
# --------------------------------------------------------------------------
def draft_limit(L: int, T: int, i: int) -> int:
    """Tokens draft token i (0-based) of a T-token draft sees when the draft is
    the last T of the L context tokens: itself and everything before it."""
    return min(max(L - T + 1 + i, 0), L)


def paged_verify(q, k_pool, v_pool, block_tables, context_lens, scale, dtype) -> np.ndarray:
    """out[s][i][h] = softmax(scale * q[s,i,h] K^T) V over the first
    draft_limit(L_s, T, i) tokens of sequence s.  q is [B][T][H_q][d] (stored
    form); returns float64 [B][T][H_q][d]; a row that sees no token is 0."""
    B, T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    scale64 = float(np.float32(scale))
    out = np.zeros((B, T, Hq, d))
    for s in range(B):
        L = int(context_lens[s])
        for g in range(Hkv):
            K = widen(k_rows(k_pool, block_tables[s], L, g), dtype)
            V = widen(v_rows(v_pool, block_tables[s], L, g), dtype)
            for i in range(T):
                lim = draft_limit(L, T, i)
                for h in range(Hq):
                    if _gqa_kv_head(h, Hq, Hkv) == g:
                        out[s, i, h], _ = attend_range(widen(q[s, i, h], dtype), K[:lim], V[:lim],
                                                       scale64)
    return out


def paged_verify_partials(q, k_pool, v_pool, block_tables, context_lens, scale, dtype,
                          partition_size: int, max_context_len: int):
    """Partition partials of paged_verify, rows ordered (s, i, h):
    o_part [B][T * H_q][n_parts][d], lse_part [B][T * H_q][n_parts]; partition p
    of draft token i covers tokens [pP, min(draft_limit, (p+1)P))."""
    B, T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    P = num_partitions(max_context_len, partition_size)
    scale64 = float(np.float32(scale))
    o_part = np.zeros((B, T * Hq, P, d))
    lse_part = np.full((B, T * Hq, P), -np.inf)
    for s in range(B):
        L = int(context_lens[s])
        for g in range(Hkv):
            K = widen(k_rows(k_pool, block_tables[s], L, g), dtype)
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
