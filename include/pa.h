/*
 * pa.h -- single-token decode attention over a paged KV cache, for MI355X (gfx950).
 *
 * The method: K and V of every cached token live in a shared pool of fixed-size
 * physical blocks of 16 tokens; a per-sequence block table maps logical block i
 * (tokens 16i .. 16i+15) to a physical block; blocks are taken from the pool
 * when they are written and several tables may point at the same physical block
 * (a shared prompt prefix).  See the pages
 *   "LLM 推理优化：KV Cache、PagedAttention 与量化" (blog.tanteng.space), §2.2, §2.3
 *   "大模型推理加速与显存黑科技 (Inference Acceleration & KV Cache)" (ialgorithm.me),
 *     §2 (attention equation), §3.2 (block-table figure), §4.2 (online softmax)
 *   "大模型推理加速：从 KV Cache 到投机采样的工程实践" (ybb.press), "主流优化策略" (GQA/MQA)
 *   "LLM推理优化实战：从KV Cache到Speculative Decoding，把延迟打下来" (jsqmd.com),
 *     KVCacheAttention listing (scale d^-0.5; new K/V appended before attending).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All pointers except `pool` descriptors are DEVICE pointers owned by the
 *    caller.  The library allocates no device memory, keeps no state between
 *    calls and is reentrant.
 *  - Every call is asynchronous on `stream` (NULL = the null stream) and never
 *    synchronises.  Argument errors are reported synchronously by the return
 *    value and nothing is launched; PA_ERR_HIP reports a failed launch.
 *  - Element dtype: PA_F32 (IEEE binary32), PA_F16 (IEEE binary16), PA_BF16
 *    (bfloat16).  q, out, the pools and new K/V rows share the pool dtype.
 *    PA_K8_F16 / PA_K8_BF16: int8 keys (see pa_write_kv_k8), 16-bit values.
 *    PA_K2_F16 / PA_K2_BF16: 2-bit keys (see pa_write_kv_k2), 16-bit values.
 *  - KV pool layout.  Both pools are arrays of tiles, one tile per (physical
 *    block, kv head), block-major then head; a tile holds the bs tokens of the
 *    block (bs = block_size, 16 or 8), bs * head_dim elements, contiguous (4 KiB
 *    for 16 tokens at head_dim 128 in a 16-bit dtype).  Token slot =
 *    physical_block * bs + offset.  Inside a tile:
 *      k_pool  [num_blocks][num_kv_heads][head_dim / x][bs][x], x = 16 bytes /
 *              element size (8 for f16/bf16, 4 for f32): each token row is cut
 *              into 16-byte chunks and the tile stores chunk 0 of its bs tokens,
 *              then chunk 1, ...;
 *      v_pool  [num_blocks][num_kv_heads][head_dim][bs]: the tile stores
 *              element 0 of its bs tokens, then element 1, ...
 *    These orders make every operand of the decode kernel's matrix products a
 *    contiguous per-lane load.  An int8 key pool (PA_K8_*) has the same K
 *    order with x = 16: [num_blocks][num_kv_heads][head_dim / 16][16][16]
 *    (2 KiB tiles of 16 tokens at head_dim 128); its V pool is the 16-bit one.
 *    A 2-bit key pool (PA_K2_*) holds bs * head_dim / 16 32-bit words per tile
 *    (512 bytes for 16 tokens at head_dim 128), as uint32
 *    [num_blocks][num_kv_heads][4][bs][head_dim / 64]: channel c of the token
 *    at offset o is the 2-bit field at bit 2 * (4 * ((c / 32) % 2) + (c % 8) / 2)
 *    + 16 * (c % 2) of word [(c % 32) / 8][o][c / 64].  So word w of group q
 *    holds channels 32 j + 8 q + e of one token for j = 2w, 2w + 1 and e = 0..7,
 *    the two of a pair (e = 2i, 2i + 1) 16 bits apart: one shift and one mask
 *    give the pair as the low bits of two 16-bit halves.
 *  - Block tables: int32 [num_seqs][max_blocks_per_seq], row-major.  Entry j of
 *    row s is the physical block of tokens bs*j .. bs*j + bs-1 of sequence s.
 *    Only the first ceil(context_lens[s] / bs) entries of a row are read.
 *  - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads)
 *    (contiguous groups; num_q_heads == num_kv_heads is MHA, num_kv_heads == 1 MQA).
 *  - Device-side data are not validated (that would need a synchronisation):
 *    a physical id outside [0, num_blocks) is clamped into range and a context
 *    length is clamped into [0, max_context_len], so a bad table yields a wrong
 *    result but never an out-of-bounds access.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad head ratio, ... */
  PA_ERR_UNSUPPORTED = -2, /* dtype, head_dim or block_size outside what is built */
  PA_ERR_MISALIGNED = -3,  /* a device pointer is not 16-byte aligned */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than pa_decode_workspace_bytes */
  PA_ERR_HIP = -5,         /* a kernel launch failed */
  PA_ERR_NO_SPACE = -6     /* block manager: the pool has too few free + cached blocks */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  /* Quantised keys: K is int8 with float32 per-(KV head, channel) scales, V,
   * q and out are 16-bit (f16 or bf16).  Used by pa_write_kv_k8 and
   * pa_decode_k8; the plain pa_write_kv / pa_decode calls reject them. */
  PA_K8_F16 = 3,
  PA_K8_BF16 = 4,
  /* 2-bit keys with float32 per-(KV head, channel) scales and zero points, V,
   * q and out 16-bit.  Used by pa_write_kv_k2 and pa_decode_k2 only. */
  PA_K2_F16 = 5,
  PA_K2_BF16 = 6
} pa_dtype;

/* Host-side description of a KV pool.  block_size is 16 (the pages' default)
 * or 8 (the smaller blocks §2.2 of the blog.tanteng.space page mentions for
 * 70B models); head_dim is 64 or 128. */
typedef struct pa_pool_desc {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* a pa_dtype value */
} pa_pool_desc;

/* Fill every element of both pools: fill = 0 writes +0.0, fill = 1 writes a
 * quiet NaN (used to prove that unreferenced blocks are never read; an int8
 * key pool gets -128, a code no write produces; a 2-bit key pool, where every
 * bit pattern is a code, gets all ones, code 3).  Meant for a pool just taken
 * from the allocator, before any block of it is written (the fixed-capacity
 * block pool of §2.3 of the blog.tanteng.space page). */
pa_status pa_init_pool(const pa_pool_desc* pool, void* k_pool, void* v_pool, int32_t fill,
                       hipStream_t stream);

/* KV append: for each of num_tokens new tokens i, copy k_new[i] and v_new[i]
 * ([num_kv_heads][head_dim] each, pool dtype, so k_new is [num_tokens][H_kv][d])
 * bit for bit into slot slot_mapping[i] = physical * bs + offset of both pools,
 * in the tile layouts above.
 * A negative slot skips the token; slots >= num_blocks * bs are also skipped.
 * Two tokens with the same slot race (the caller's contract).  This is the step
 * that puts the new token's K/V into the cache before attention, as the
 * KVCacheAttention listing of the jsqmd.com page does with its concatenation. */
pa_status pa_write_kv(const pa_pool_desc* pool, void* k_pool, void* v_pool, const void* k_new,
                      const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                      hipStream_t stream);

/* Bytes of workspace pa_decode needs for split-context partials: float32
 * o_part[num_seqs][num_q_heads][n_parts][head_dim] followed by float32
 * lse_part[num_seqs][num_q_heads][n_parts], n_parts = ceil(max_context_len /
 * partition_size).  0 when partition_size is 0 (single phase) and on bad
 * arguments. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

/* Decode attention for one query token per sequence:
 *   out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s
 * over the context_lens[s] tokens the block table of s addresses (the equation
 * of §2 of the ialgorithm.me page; the gather of its §3.2 figure).  q and out
 * are [num_seqs][num_q_heads][head_dim] in the pool dtype; out is rounded to
 * nearest-even from float32 accumulators.  A zero-length context gives a zero
 * row.
 *
 * partition_size == 0: single phase, out is written.
 * partition_size  > 0 (a multiple of 16): the context of each sequence is cut
 *   into partitions of partition_size tokens; partition p of (s, h) writes
 *   o_part = its own normalised attention output and lse_part = ln sum exp of
 *   its logits (-inf and a zero row for an empty partition) into `workspace`
 *   (layout: pa_decode_workspace_bytes); `out` is not touched and may be NULL.
 *   pa_reduce then merges the partials into out.
 * max_context_len bounds every context length and must not exceed
 * bs * max_blocks_per_seq.  Partition sizes are multiples of 16 tokens for
 * either block size. */
pa_status pa_decode(const pa_pool_desc* pool, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* out, hipStream_t stream);

/* The verify step of speculative decoding: T = num_query_tokens draft tokens
 * per sequence are scored in one call (the target model checks all of a draft
 * model's candidates in one forward pass: §6.2 of the blog.tanteng.space page,
 * §5.1 of the ialgorithm.me page; drafts of 4-8 tokens in "投机采样" of the
 * ybb.press page).  The T draft tokens are the last T tokens of each context:
 * their K/V are already in the pool (pa_write_kv) and context_lens[s] counts
 * them.  Draft token i (0-based) of sequence s attends causally, to the tokens
 * [0, context_lens[s] - T + 1 + i):
 *   out[s][i][h] = softmax(scale * q[s][i][h] . K_s[0 .. lim)^T) V_s[0 .. lim).
 * So row i equals what pa_decode returns for that token when the sequence is
 * decoded one token at a time.  A row with lim <= 0 is zero.  q and out are
 * [num_seqs][T][num_q_heads][head_dim] in the pool dtype; 1 <= T <= 256.  T = 1
 * is pa_decode.  Split mode works as in pa_decode with T * num_q_heads rows
 * per sequence: size the workspace with pa_decode_workspace_bytes(num_seqs,
 * T * num_q_heads, ...) and merge with pa_reduce(..., T * num_q_heads, ...).
 * The T * G rows of one KV head (G = num_q_heads / num_kv_heads) are computed
 * together, so each K/V tile is read once for all draft tokens. */
pa_status pa_verify_decode(const pa_pool_desc* pool, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                           int32_t max_context_len, float scale, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, void* out,
                           hipStream_t stream);

/* Log-sum-exp merge of the partials pa_decode wrote into `workspace` (same
 * num_seqs, num_q_heads, head_dim, max_context_len and partition_size):
 *   M = max_p lse_p,  LSE = M + ln sum_p exp(lse_p - M),
 *   out[s][h] = sum_p exp(lse_p - LSE) o_p,
 * over the ceil(context_lens[s] / partition_size) partitions sequence s has.
 * Exact because the softmax normaliser can be streamed (§4.2 of the
 * ialgorithm.me page).  out is [num_seqs][num_q_heads][head_dim] in out_dtype.
 * workspace_bytes is the size of the workspace buffer: PA_ERR_WORKSPACE when it
 * is below pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 * max_context_len, partition_size) (the merge would read past it). */
pa_status pa_reduce(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_context_len, int32_t partition_size, int32_t out_dtype, void* out,
                    hipStream_t stream);

/* The gather indices pa_decode uses, computed by the same device function:
 * slot_ids[s][t] = block_tables[s][t / bs] * bs + t % bs for t < context_lens[s]
 * (after the same clamping), -1 for context_lens[s] <= t < max_context_len,
 * with bs = block_size (16 or 8).  slot_ids is int64 [num_seqs][max_context_len].
 * Used to check the block-table arithmetic bit for bit (the worked example of
 * §3.2 of the ialgorithm.me page).  num_blocks is the pool size used for
 * clamping. */
pa_status pa_debug_slot_ids(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t num_blocks, int32_t block_size,
                            int64_t* slot_ids, hipStream_t stream);

/* Split decode of a batch whose block tables all start with the same
 * prefix_tokens / bs physical blocks (a shared system prompt: §2.3 of the
 * blog.tanteng.space page, blocks referenced by several tables).  The result
 * is exactly pa_decode's (or pa_decode_k8's / pa_decode_k2's) in split mode
 * with partition_size: the same partials in the same workspace layout, merged
 * afterwards by pa_reduce with the same partition_size.  The partitions of the
 * prefix are computed once per KV head for the query rows of every sequence
 * together (each prefix tile is read from memory once for the batch instead of
 * once per sequence); the rest of each context is computed per sequence as
 * pa_decode does.
 *
 * Any pool type: k_scale is the int8 or 2-bit keys' float32 [H_kv][d] scales
 * (steps), k_zero the 2-bit keys' zero points, both as for pa_decode_k8 /
 * pa_decode_k2 and null for the other pools (PA_ERR_INVALID_ARG when a
 * quantised pool lacks them, PA_ERR_UNSUPPORTED when a plain pool gets them).
 * prefix_tokens: a positive multiple of partition_size, at most
 * max_context_len; partition_size > 0, a multiple of 16.  One query token per
 * sequence (q [num_seqs][num_q_heads][head_dim]).  Caller's contract on device
 * data (not checked): every table's first prefix_tokens / bs entries equal
 * table row 0's, and every context_lens[s] >= prefix_tokens; otherwise the
 * prefix partitions use row 0's blocks and all prefix_tokens tokens anyway (a
 * wrong result, never an out-of-bounds access). */
pa_status pa_decode_shared_prefix(const pa_pool_desc* pool, const void* q, const void* k_pool,
                                  const void* v_pool, const float* k_scale, const float* k_zero,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len, float scale,
                                  int32_t prefix_tokens, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Quantised key cache (§4.2 of the blog.tanteng.space page: keys quantised
 * per channel, values kept in 16-bit; "KV Cache量化" of the ybb.press page:
 * INT8 caches, per-channel keys because key channels are unevenly scaled).
 * The pool dtype is PA_K8_F16 or PA_K8_BF16.  k_scale is float32
 * [num_kv_heads][head_dim] in device memory: the static scale of each key
 * channel (e.g. its calibrated max |k| / 127), positive and finite.
 *
 * pa_write_kv_k8: as pa_write_kv, but each key element k of channel c becomes
 *   code = clamp(rint(k / k_scale[g][c]), -127, 127)
 * (float32 division rounded to nearest, ties to even), stored as int8 in the K
 * layout above; V rows are copied bit for bit.  k_new and v_new are
 * [num_tokens][H_kv][d] in the 16-bit type; key rows must be finite.
 *
 * pa_decode_k8: pa_verify_decode (num_query_tokens = 1 is pa_decode) over the
 * dequantised keys code * k_scale[g][c]; q and out in the 16-bit type, split
 * mode and pa_reduce as there.  A K tile is half the bytes of a 16-bit one:
 * 3/4 of the KV traffic per token. */
pa_status pa_write_kv_k8(const pa_pool_desc* pool, void* k_pool, void* v_pool, const float* k_scale,
                         const void* k_new, const void* v_new, const int64_t* slot_mapping,
                         int32_t num_tokens, hipStream_t stream);
pa_status pa_decode_k8(const pa_pool_desc* pool, const void* q, const void* k_pool,
                       const void* v_pool, const float* k_scale, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_query_tokens, int32_t num_q_heads, int32_t max_context_len,
                       float scale, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, void* out, hipStream_t stream);

/* 2-bit key cache, asymmetric per channel (KIVI as §4.2 of the
 * blog.tanteng.space page describes it: keys at 2 bits per channel, values kept
 * in 16-bit; asymmetric quantisation as "KV Cache量化" of the ybb.press page
 * says).  The pool dtype is PA_K2_F16 or PA_K2_BF16.  k_scale and k_zero are
 * float32 [num_kv_heads][head_dim] in device memory, 16-byte aligned: the
 * static step s and zero point z of each key channel (e.g. a calibrated
 * minimum z and s = (maximum - minimum) / 3), finite, s >= 0.
 *
 * pa_write_kv_k2: as pa_write_kv, but each key element k of channel c becomes
 *   u = (k - z) / s  (float32 subtraction and division, round to nearest),
 *   code = rint(min(max(u, 0), 3))  (ties to even; min/max ignore a NaN, so
 *   s = 0 gives code 0 at or below z and 3 above it),
 * stored in the 2-bit layout above (a written token's key words are replaced
 * whole); V rows are copied bit for bit.  k_new and v_new are
 * [num_tokens][H_kv][d] in the 16-bit type; key rows must be finite.
 *
 * pa_decode_k2: pa_verify_decode (num_query_tokens = 1 is pa_decode) over the
 * dequantised keys z + s * code; q and out in the 16-bit type, split mode and
 * pa_reduce as there (partials include the zero points' contribution to the
 * log-sum-exp).  A K tile is 1/8 of a 16-bit one: 9/16 of the KV traffic per
 * token. */
pa_status pa_write_kv_k2(const pa_pool_desc* pool, void* k_pool, void* v_pool, const float* k_scale,
                         const float* k_zero, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int32_t num_tokens, hipStream_t stream);
pa_status pa_decode_k2(const pa_pool_desc* pool, const void* q, const void* k_pool,
                       const void* v_pool, const float* k_scale, const float* k_zero,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_query_tokens,
                       int32_t num_q_heads, int32_t max_context_len, float scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes, void* out,
                       hipStream_t stream);

/* Copy whole blocks inside the pool: for each i < num_pairs, block
 * src_dst[2i + 1] of both pools becomes a copy of block src_dst[2i] (every KV
 * head, K and V).  This is the copy of a copy-on-write (§2.3 (2) of the
 * blog.tanteng.space page: a sequence that writes into a block it shares gets
 * its own copy first).  src_dst is int32 [num_pairs][2] in device
 * memory.  A pair with an id outside [0, num_blocks) or with src == dst is
 * skipped.  Destinations must be distinct and must not be sources of other
 * pairs of the same call (they would race). */
pa_status pa_copy_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                         const int32_t* src_dst, int32_t num_pairs, hipStream_t stream);

/* Swap support (preemption, §2.3 (1) of the blog.tanteng.space page: a full pool
 * moves a request's blocks out to host memory and back later).
 * pa_gather_blocks packs blocks block_ids[0 .. n) of both pools contiguously:
 * block i goes to k_dst / v_dst at byte offset i * block_bytes, block_bytes =
 * num_kv_heads * bs * head_dim * element size of that pool (the pool's own
 * tile order; 1 byte for int8 keys, 1/4 byte for 2-bit keys).
 * pa_scatter_blocks is the inverse: k_src / v_src block i goes to pool block
 * block_ids[i].  block_ids is int32 in device memory; ids outside the pool are
 * skipped.  The packed buffers must be device-accessible (device memory, or
 * pinned host memory) and 16-byte aligned; the caller moves them between host
 * and device.  Scatter destinations must be distinct. */
pa_status pa_gather_blocks(const pa_pool_desc* pool, const void* k_pool, const void* v_pool,
                           const int32_t* block_ids, int32_t n, void* k_dst, void* v_dst,
                           hipStream_t stream);
pa_status pa_scatter_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                            const int32_t* block_ids, int32_t n, const void* k_src,
                            const void* v_src, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): pa_decode
 * in split mode followed by pa_reduce, with the partials in a fixed device
 * array of PA_STATIC_SCRATCH_BYTES inside the library instead of a caller
 * workspace.  Arguments as pa_decode's (16-bit or float32 pools; quantised
 * pools are PA_ERR_UNSUPPORTED), partition_size > 0, out written as by
 * pa_reduce; the result is the same bits as pa_decode + pa_reduce with the
 * same partition_size.  PA_ERR_WORKSPACE when pa_decode_workspace_bytes for
 * these arguments exceeds PA_STATIC_SCRATCH_BYTES.  Nothing is allocated: each
 * GPU the library runs on holds one copy of the array until the process ends
 * (its address is looked up on the first call made with that device current).
 * Every call on a GPU uses that GPU's one array, so calls that overlap on one
 * GPU (on different streams, or from several threads) race; calls on one
 * stream are ordered and safe.  The array keeps the last call's partials; no
 * call reads a partial it did not write. */
#define PA_STATIC_SCRATCH_BYTES (32u << 20)
pa_status pa_decode_split_static(const pa_pool_desc* pool, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 float scale, int32_t partition_size, void* out,
                                 hipStream_t stream);

/* Measurement probes (not part of the attention): the achievable read rates
 * the decode kernel's HBM roofline is read against.  Decode attention is bound
 * by moving K/V from HBM to the compute units (§4.1 of the ialgorithm.me page,
 * §3.1 of the blog.tanteng.space page), so these read exactly that and compute
 * nothing.  Each folds what it reads into one XOR word per wavefront, written
 * to `sink` (device memory, caller-owned), so no load can be dropped.
 *
 * pa_probe_read: reads `bytes` (a positive multiple of 16) at `src` (16-byte
 *   aligned) with 16-byte streaming loads, each wavefront whole contiguous
 *   4 KiB runs, over sink_words / 4 workgroups of 256 threads; sink holds
 *   sink_words 32-bit words (a positive multiple of 4).
 * pa_probe_read_tiles: reads the K and V tiles pa_decode (unsplit) reads for the
 *   same pool, tables and lengths, in its order and with its loads: one
 *   workgroup of 8 wavefronts per (sequence, KV head), wavefront w reads the
 *   16-token blocks w, w + 8, ... through the block table.  16-bit pools of
 *   16-token blocks, head_dim 64 or 128; physical ids and lengths are clamped
 *   as in pa_decode.  sink holds sink_words 32-bit words, at least
 *   num_seqs * num_kv_heads * 8 (one per wavefront); fewer is
 *   PA_ERR_INVALID_ARG. */
pa_status pa_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_words,
                        hipStream_t stream);
pa_status pa_probe_read_tiles(const pa_pool_desc* pool, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, uint32_t* sink, int32_t sink_words,
                              hipStream_t stream);

/* Static, NUL-terminated name of a status code. */
const char* pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
