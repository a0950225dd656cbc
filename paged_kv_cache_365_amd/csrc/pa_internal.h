// Host-side launch interfaces between the C-ABI front end (pa_api.hip) and the
// kernel translation units.  Arguments are validated by the front end before
// any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;  // quantised keys: float32 [H_kv][d] channel scales (steps); else null
  const float* k_zero;   // 2-bit keys: float32 [H_kv][d] channel zero points; else null
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_query_tokens;  // query tokens per sequence: 1 (decode) or T (verify)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_blocks;
  int32_t block_size;        // tokens per physical block: 16 or 8
  int32_t max_context_len;
  int32_t dtype;
  float scale;
  int32_t partition_tokens;  // tokens per partition (a multiple of 16)
  int32_t num_parts;         // partitions per sequence in the grid
  int32_t part_stride;       // partitions per row in the workspace (>= part_offset + num_parts)
  int32_t part_offset;       // first partition the grid computes
  // shared-prefix launches: the prefix role covers partitions [0, shared_parts)
  // of the shared_tokens-token prefix (set by the launcher: shared_units)
  int32_t shared_parts;
  int32_t shared_tokens;
  int32_t shared_units;
  bool write_partials;       // true: o_part/lse_part into the workspace; false: out
  float* o_part;
  float* lse_part;
  void* out;
};

// Launch the decode kernel chosen for (dtype, head_dim).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Shared-prefix split launch (any pool type, one query token).
hipError_t launch_decode_shared_prefix(const DecodeArgs& a, hipStream_t stream);

struct ReduceArgs {
  const float* o_part;
  const float* lse_part;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t max_context_len;
  int32_t partition_tokens;
  int32_t num_parts;
  int32_t dtype;
  void* out;
};
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);

hipError_t launch_fill(void* dst, size_t bytes16, uint32_t pattern, hipStream_t stream);

hipError_t launch_write_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t row_bytes,
                           int32_t elem_bytes, hipStream_t stream);

struct BlockMoveArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int32_t* src_ids;  // null: pair index
  int32_t src_stride;
  int32_t src_limit;       // blocks in the source buffers
  const int32_t* dst_ids;  // null: pair index
  int32_t dst_stride;
  int32_t dst_limit;
  int32_t num_pairs;
  size_t k_block_bytes;    // bytes of one block of the K buffers (a multiple of 16)
  size_t v_block_bytes;    // bytes of one block of the V buffers (a multiple of 16)
  bool skip_equal;
};
hipError_t launch_block_move(const BlockMoveArgs& a, hipStream_t stream);

hipError_t launch_write_kv_k8(void* k_pool, void* v_pool, const float* k_scale, const void* k_new,
                              const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_dim, int32_t dtype, hipStream_t stream);

hipError_t launch_write_kv_k2(void* k_pool, void* v_pool, const float* k_scale, const float* k_zero,
                              const void* k_new, const void* v_new, const int64_t* slot_mapping,
                              int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                              hipStream_t stream);

hipError_t launch_slot_ids(const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           int32_t num_blocks, int32_t block_size, int64_t* slot_ids,
                           hipStream_t stream);

}  // namespace pa
