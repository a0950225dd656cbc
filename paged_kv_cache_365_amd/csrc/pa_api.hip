// C-ABI front end: argument validation, workspace sizing, kernel selection.
// Nothing here allocates device memory or synchronises.
#include <limits.h>

#include <mutex>

#include "pa_common.h"
#include "pa_internal.h"

namespace {

constexpr int kMaxQueryTokens = 256;   // draft tokens per sequence in one verify call

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// bytes of one V element (also of q, out and new K/V rows); 0 for unknown
int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16:
    case PA_BF16:
    case PA_K8_F16:
    case PA_K8_BF16:
    case PA_K2_F16:
    case PA_K2_BF16: return 2;
    default: return 0;
  }
}

bool is_k8(int32_t dtype) { return dtype == PA_K8_F16 || dtype == PA_K8_BF16; }
bool is_k2(int32_t dtype) { return dtype == PA_K2_F16 || dtype == PA_K2_BF16; }
bool is_quantized(int32_t dtype) { return is_k8(dtype) || is_k2(dtype); }

// bits of one K element in the pool
int k_elem_bits(int32_t dtype) { return is_k2(dtype) ? 2 : (is_k8(dtype) ? 8 : 8 * elem_bytes(dtype)); }

pa_status check_pool(const pa_pool_desc* pool) {
  if (!pool) return PA_ERR_INVALID_ARG;
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (pool->block_size != 16 && pool->block_size != 8) return PA_ERR_UNSUPPORTED;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (elem_bytes(pool->dtype) == 0) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

size_t block_elems(const pa_pool_desc* pool) {
  return static_cast<size_t>(pool->num_kv_heads) * pool->block_size * pool->head_dim;
}
// bytes of one block of the K pool (every KV head): a multiple of 16
size_t k_block_bytes(const pa_pool_desc* pool) {
  return block_elems(pool) * k_elem_bits(pool->dtype) / 8;
}
size_t k_pool_bytes(const pa_pool_desc* pool) { return pool->num_blocks * k_block_bytes(pool); }
size_t v_pool_bytes(const pa_pool_desc* pool) {
  return pool->num_blocks * block_elems(pool) * elem_bytes(pool->dtype);
}

int32_t num_parts_for(int32_t max_context_len, int32_t partition_size) {
  const int64_t n = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
  return static_cast<int32_t>(n < 1 ? 1 : n);
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_MISALIGNED: return "PA_ERR_MISALIGNED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_NO_SPACE: return "PA_ERR_NO_SPACE";
  }
  return "PA_ERR_UNKNOWN";
}

pa_status pa_init_pool(const pa_pool_desc* pool, void* k_pool, void* v_pool, int32_t fill,
                       hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (!k_pool || !v_pool || (fill != 0 && fill != 1)) return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16)) return PA_ERR_MISALIGNED;
  uint32_t v_pattern = 0u, k_pattern = 0u;
  if (fill == 1) {
    const bool f16 = pool->dtype == PA_F16 || pool->dtype == PA_K8_F16 || pool->dtype == PA_K2_F16;
    v_pattern = pool->dtype == PA_F32 ? 0x7FC00000u : (f16 ? 0x7E007E00u : 0x7FC07FC0u);
    k_pattern = is_k8(pool->dtype) ? 0x80808080u : v_pattern;  // int8 -128: no write makes it
    if (is_k2(pool->dtype)) k_pattern = 0xFFFFFFFFu;  // every 2-bit pattern is a code: all 3s
  }
  hipError_t e = pa::launch_fill(k_pool, k_pool_bytes(pool), k_pattern, stream);
  if (e == hipSuccess) e = pa::launch_fill(v_pool, v_pool_bytes(pool), v_pattern, stream);
  return from_hip(e);
}

pa_status pa_write_kv(const pa_pool_desc* pool, void* k_pool, void* v_pool, const void* k_new,
                      const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                      hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (is_quantized(pool->dtype)) return PA_ERR_UNSUPPORTED;  // pa_write_kv_k8 / pa_write_kv_k2
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(slot_mapping, 8))
    return PA_ERR_MISALIGNED;
  const int row_bytes = pool->head_dim * elem_bytes(pool->dtype);
  return from_hip(pa::launch_write_kv(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens,
                                      pool->num_blocks, pool->block_size, pool->num_kv_heads,
                                      row_bytes, elem_bytes(pool->dtype), stream));
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return 0;
  const size_t parts = static_cast<size_t>(num_parts_for(max_context_len, partition_size));
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * parts;
  return rows * head_dim * sizeof(float) + rows * sizeof(float);
}

}  // extern "C"

namespace {

// pa_decode and pa_verify_decode: T query tokens per sequence (T = 1: decode).
pa_status decode_common(const pa_pool_desc* pool, const void* q, const void* k_pool,
                        const void* v_pool, const float* k_scale, const float* k_zero,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_query_tokens,
                        int32_t num_q_heads, int32_t max_context_len, float scale,
                        int32_t partition_size, void* workspace, size_t workspace_bytes, void* out,
                        hipStream_t stream, int32_t prefix_tokens = 0) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (is_quantized(pool->dtype) != (k_scale != nullptr) || is_k2(pool->dtype) != (k_zero != nullptr)) {
    // quantised keys need their scales (2-bit keys their zero points too);
    // other pools take none
    return is_quantized(pool->dtype) ? PA_ERR_INVALID_ARG : PA_ERR_UNSUPPORTED;
  }
  if (num_seqs <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_query_tokens < 1 || num_query_tokens > kMaxQueryTokens) return PA_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * pool->block_size)
    return PA_ERR_INVALID_ARG;
  if (partition_size < 0 || partition_size % pa::kStep != 0) return PA_ERR_INVALID_ARG;
  // one workgroup per 16 (query token, head) rows at most, per KV head, sequence
  // and partition: the one-dimensional grid must count them in 31 bits
  const int64_t rows = static_cast<int64_t>(num_query_tokens) * (num_q_heads / pool->num_kv_heads);
  const int64_t parts = partition_size > 0 ? num_parts_for(max_context_len, partition_size) : 1;
  if (static_cast<int64_t>(num_seqs) * pool->num_kv_heads * ((rows + 15) / 16) * parts > INT32_MAX)
    return PA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(block_tables, 4) ||
      !aligned(context_lens, 4) || !aligned(k_scale, 16) || !aligned(k_zero, 16))
    return PA_ERR_MISALIGNED;

  pa::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.k_zero = k_zero;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_query_tokens = num_query_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.max_context_len = max_context_len;
  a.dtype = pool->dtype;
  a.scale = scale;

  const int32_t row_heads = num_query_tokens * num_q_heads;  // output rows per sequence
  if (partition_size == 0) {
    if (!out) return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16)) return PA_ERR_MISALIGNED;
    // one partition spanning every context
    const int64_t span = (static_cast<int64_t>(max_context_len) + pa::kStep - 1) / pa::kStep *
                         pa::kStep;
    a.partition_tokens = static_cast<int32_t>(span < pa::kStep ? pa::kStep : span);
    a.num_parts = 1;
    a.part_stride = 1;
    a.write_partials = false;
    a.out = out;
  } else {
    const size_t need = pa_decode_workspace_bytes(num_seqs, row_heads, pool->head_dim,
                                                  max_context_len, partition_size);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_MISALIGNED;
    a.partition_tokens = partition_size;
    a.num_parts = num_parts_for(max_context_len, partition_size);
    a.part_stride = a.num_parts;
    a.write_partials = true;
    const size_t nrows = static_cast<size_t>(num_seqs) * row_heads * a.num_parts;
    a.o_part = static_cast<float*>(workspace);
    a.lse_part = a.o_part + nrows * pool->head_dim;
  }
  if (prefix_tokens > 0) {
    // the shared prefix is the first prefix_tokens / partition_size partitions
    a.shared_parts = prefix_tokens / partition_size;
    a.shared_tokens = prefix_tokens;
    a.part_offset = a.shared_parts;
    a.num_parts = a.part_stride - a.shared_parts;  // private partitions in the grid
    return from_hip(pa::launch_decode_shared_prefix(a, stream));
  }
  return from_hip(pa::launch_decode(a, stream));
}

}  // namespace

extern "C" {

pa_status pa_decode(const pa_pool_desc* pool, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* out, hipStream_t stream) {
  if (pool && is_quantized(pool->dtype)) return PA_ERR_UNSUPPORTED;  // pa_decode_k8 / _k2
  return decode_common(pool, q, k_pool, v_pool, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, 1, num_q_heads, max_context_len, scale,
                       partition_size, workspace, workspace_bytes, out, stream);
}

pa_status pa_verify_decode(const pa_pool_desc* pool, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                           int32_t max_context_len, float scale, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, void* out,
                           hipStream_t stream) {
  if (pool && is_quantized(pool->dtype)) return PA_ERR_UNSUPPORTED;  // pa_decode_k8 / _k2
  return decode_common(pool, q, k_pool, v_pool, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_query_tokens, num_q_heads, max_context_len,
                       scale, partition_size, workspace, workspace_bytes, out, stream);
}

pa_status pa_decode_k8(const pa_pool_desc* pool, const void* q, const void* k_pool,
                       const void* v_pool, const float* k_scale, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_query_tokens, int32_t num_q_heads, int32_t max_context_len,
                       float scale, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, void* out, hipStream_t stream) {
  if (pool && !is_k8(pool->dtype)) return PA_ERR_UNSUPPORTED;  // pa_decode / pa_verify_decode
  if (!k_scale) return PA_ERR_INVALID_ARG;
  return decode_common(pool, q, k_pool, v_pool, k_scale, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_query_tokens, num_q_heads, max_context_len,
                       scale, partition_size, workspace, workspace_bytes, out, stream);
}

pa_status pa_decode_shared_prefix(const pa_pool_desc* pool, const void* q, const void* k_pool,
                                  const void* v_pool, const float* k_scale, const float* k_zero,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len, float scale,
                                  int32_t prefix_tokens, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (partition_size <= 0 || prefix_tokens <= 0 || prefix_tokens % partition_size != 0 ||
      prefix_tokens > max_context_len)
    return PA_ERR_INVALID_ARG;
  // always split: partials into the workspace, merged by pa_reduce
  return decode_common(pool, q, k_pool, v_pool, k_scale, k_zero, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, 1, num_q_heads, max_context_len, scale,
                       partition_size, workspace, workspace_bytes, nullptr, stream, prefix_tokens);
}

pa_status pa_write_kv_k8(const pa_pool_desc* pool, void* k_pool, void* v_pool, const float* k_scale,
                         const void* k_new, const void* v_new, const int64_t* slot_mapping,
                         int32_t num_tokens, hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (!is_k8(pool->dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_scale || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(slot_mapping, 8) || !aligned(k_scale, 4))
    return PA_ERR_MISALIGNED;
  return from_hip(pa::launch_write_kv_k8(k_pool, v_pool, k_scale, k_new, v_new, slot_mapping,
                                         num_tokens, pool->num_blocks, pool->block_size,
                                         pool->num_kv_heads, pool->head_dim, pool->dtype, stream));
}

pa_status pa_decode_k2(const pa_pool_desc* pool, const void* q, const void* k_pool,
                       const void* v_pool, const float* k_scale, const float* k_zero,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_query_tokens,
                       int32_t num_q_heads, int32_t max_context_len, float scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes, void* out,
                       hipStream_t stream) {
  if (pool && !is_k2(pool->dtype)) return PA_ERR_UNSUPPORTED;  // pa_decode / _k8 / verify
  if (!k_scale || !k_zero) return PA_ERR_INVALID_ARG;
  return decode_common(pool, q, k_pool, v_pool, k_scale, k_zero, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_query_tokens, num_q_heads, max_context_len,
                       scale, partition_size, workspace, workspace_bytes, out, stream);
}

pa_status pa_write_kv_k2(const pa_pool_desc* pool, void* k_pool, void* v_pool, const float* k_scale,
                         const float* k_zero, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (!is_k2(pool->dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_scale || !k_zero || !k_new || !v_new || !slot_mapping)
    return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(slot_mapping, 8) || !aligned(k_scale, 16) || !aligned(k_zero, 16))
    return PA_ERR_MISALIGNED;
  return from_hip(pa::launch_write_kv_k2(k_pool, v_pool, k_scale, k_zero, k_new, v_new,
                                         slot_mapping, num_tokens, pool->num_blocks,
                                         pool->block_size, pool->num_kv_heads, pool->head_dim,
                                         pool->dtype, stream));
}

pa_status pa_reduce(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_context_len, int32_t partition_size, int32_t out_dtype, void* out,
                    hipStream_t stream) {
  if (!workspace || !context_lens || !out) return PA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || num_q_heads <= 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if (partition_size <= 0 || partition_size % pa::kStep != 0) return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (elem_bytes(out_dtype) == 0 || is_quantized(out_dtype)) return PA_ERR_UNSUPPORTED;
  if (workspace_bytes < pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                                  partition_size))
    return PA_ERR_WORKSPACE;
  if (!aligned(workspace, 16) || !aligned(out, 16) || !aligned(context_lens, 4))
    return PA_ERR_MISALIGNED;
  // one 64-lane wavefront per 32 output columns of a row: the threads must fit a 1-D grid
  if (static_cast<int64_t>(num_seqs) * num_q_heads * (head_dim / 32) * 64 > INT32_MAX)
    return PA_ERR_UNSUPPORTED;
  pa::ReduceArgs a{};
  a.num_parts = num_parts_for(max_context_len, partition_size);
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * a.num_parts;
  a.o_part = static_cast<const float*>(workspace);
  a.lse_part = a.o_part + rows * head_dim;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.max_context_len = max_context_len;
  a.partition_tokens = partition_size;
  a.dtype = out_dtype;
  a.out = out;
  return from_hip(pa::launch_reduce(a, stream));
}

pa_status pa_copy_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                         const int32_t* src_dst, int32_t num_pairs, hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !src_dst) return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(src_dst, 4)) return PA_ERR_MISALIGNED;
  pa::BlockMoveArgs a{};
  a.src_k = k_pool;
  a.src_v = v_pool;
  a.dst_k = k_pool;
  a.dst_v = v_pool;
  a.src_ids = src_dst;
  a.src_stride = 2;
  a.src_limit = pool->num_blocks;
  a.dst_ids = src_dst + 1;
  a.dst_stride = 2;
  a.dst_limit = pool->num_blocks;
  a.num_pairs = num_pairs;
  a.k_block_bytes = k_block_bytes(pool);
  a.v_block_bytes = block_elems(pool) * elem_bytes(pool->dtype);
  a.skip_equal = true;
  return from_hip(pa::launch_block_move(a, stream));
}

pa_status pa_gather_blocks(const pa_pool_desc* pool, const void* k_pool, const void* v_pool,
                           const int32_t* block_ids, int32_t n, void* k_dst, void* v_dst,
                           hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_ids || !k_dst || !v_dst) return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_dst, 16) || !aligned(v_dst, 16) ||
      !aligned(block_ids, 4))
    return PA_ERR_MISALIGNED;
  pa::BlockMoveArgs a{};
  a.src_k = k_pool;
  a.src_v = v_pool;
  a.dst_k = k_dst;
  a.dst_v = v_dst;
  a.src_ids = block_ids;
  a.src_stride = 1;
  a.src_limit = pool->num_blocks;
  a.dst_ids = nullptr;
  a.dst_stride = 1;
  a.dst_limit = n;
  a.num_pairs = n;
  a.k_block_bytes = k_block_bytes(pool);
  a.v_block_bytes = block_elems(pool) * elem_bytes(pool->dtype);
  a.skip_equal = false;
  return from_hip(pa::launch_block_move(a, stream));
}

pa_status pa_scatter_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                            const int32_t* block_ids, int32_t n, const void* k_src,
                            const void* v_src, hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_ids || !k_src || !v_src) return PA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_src, 16) || !aligned(v_src, 16) ||
      !aligned(block_ids, 4))
    return PA_ERR_MISALIGNED;
  pa::BlockMoveArgs a{};
  a.src_k = k_src;
  a.src_v = v_src;
  a.dst_k = k_pool;
  a.dst_v = v_pool;
  a.src_ids = nullptr;
  a.src_stride = 1;
  a.src_limit = n;
  a.dst_ids = block_ids;
  a.dst_stride = 1;
  a.dst_limit = pool->num_blocks;
  a.num_pairs = n;
  a.k_block_bytes = k_block_bytes(pool);
  a.v_block_bytes = block_elems(pool) * elem_bytes(pool->dtype);
  a.skip_equal = false;
  return from_hip(pa::launch_block_move(a, stream));
}

pa_status pa_debug_slot_ids(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t num_blocks, int32_t block_size,
                            int64_t* slot_ids, hipStream_t stream) {
  if (!block_tables || !context_lens || !slot_ids) return PA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (block_size != 16 && block_size != 8) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PA_ERR_INVALID_ARG;
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(slot_ids, 8))
    return PA_ERR_MISALIGNED;
  if (max_context_len == 0) return PA_OK;
  return from_hip(pa::launch_slot_ids(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                      max_context_len, num_blocks, block_size, slot_ids, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Split decode with no allocation: the partials live in a fixed device array.
// ---------------------------------------------------------------------------
// One copy per GPU the library runs on, held until the process ends.  Host
// code never passes `scratch` itself to a kernel or a copy: its host-side name
// is not a device address.  The address comes from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
pa_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_split_static(const pa_pool_desc* pool, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 float scale, int32_t partition_size, void* out,
                                 hipStream_t stream) {
  pa_status st = check_pool(pool);
  if (st != PA_OK) return st;
  if (is_quantized(pool->dtype)) return PA_ERR_UNSUPPORTED;
  if (partition_size <= 0 || partition_size % pa::kStep != 0 || !out) return PA_ERR_INVALID_ARG;
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, pool->head_dim,
                                                max_context_len, partition_size);
  if (need == 0) return PA_ERR_INVALID_ARG;
  if (need > PA_STATIC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != PA_OK) return st;
  // every partial the merge reads is written by the decode launch first: nothing
  // left in the array by an earlier call is read
  st = pa_decode(pool, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                 num_q_heads, max_context_len, scale, partition_size, ws, need, nullptr, stream);
  if (st != PA_OK) return st;
  return pa_reduce(ws, need, context_lens, num_seqs, num_q_heads, pool->head_dim, max_context_len,
                   partition_size, pool->dtype, out, stream);
}

}  // extern "C"
