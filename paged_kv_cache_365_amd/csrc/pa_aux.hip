// The small kernels around decode: the log-sum-exp merge of partition
// partials, pool fill, KV append and the debug slot-id gather.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// pa_reduce: one workgroup per (sequence, query head), one thread per column.
// The partition results are re-weighted by their share of the softmax mass:
// with M = max lse_p, weight_p = exp(lse_p - M) / sum_q exp(lse_q - M).  This
// is the same streaming-normaliser identity that makes the online softmax exact
// (§4.2 of the ialgorithm.me page).  Partitions are visited in order.
// ---------------------------------------------------------------------------
template <class Tr>
__global__ __launch_bounds__(128) void reduce_kernel(ReduceArgs a) {
  extern __shared__ float sm_w[];  // [num_parts] weights
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int c = threadIdx.x;
  const int L = pa_clamp_len(a.context_lens[s], a.max_context_len);
  const int nv = (L + a.partition_tokens - 1) / a.partition_tokens;  // live partitions
  const size_t r = static_cast<size_t>(s) * a.num_q_heads + h;
  const float* lse = a.lse_part + r * a.num_parts;

  float M = -INFINITY;
  for (int p = 0; p < nv; ++p) M = fmaxf(M, lse[p]);
  float o = 0.f;
  if (M != -INFINITY) {
    float sum = 0.f;
    for (int p = threadIdx.x; p < nv; p += blockDim.x) sm_w[p] = __expf(lse[p] - M);
    __syncthreads();
    for (int p = 0; p < nv; ++p) sum += sm_w[p];
    const float inv = 1.f / sum;
    if (c < a.head_dim) {
      const float* op = a.o_part + r * a.num_parts * a.head_dim + c;
      float acc = 0.f;
      for (int p = 0; p < nv; ++p) acc = fmaf(sm_w[p], op[static_cast<size_t>(p) * a.head_dim], acc);
      o = acc * inv;
    }
  }
  if (c < a.head_dim) Tr::store(a.out, r * a.head_dim + c, o);
}

template <class Tr>
hipError_t launch_reduce_t(const ReduceArgs& a, hipStream_t stream) {
  dim3 grid(a.num_q_heads, a.num_seqs);
  const int threads = a.head_dim <= 64 ? 64 : 128;
  const size_t lds = static_cast<size_t>(a.num_parts) * sizeof(float);
  hipLaunchKernelGGL(reduce_kernel<Tr>, grid, dim3(threads), lds, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fill: 16-byte stores of a repeated 32-bit pattern
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_kernel(uint4* dst, size_t n16, uint32_t pattern) {
  const uint4 v = make_uint4(pattern, pattern, pattern, pattern);
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = v;
}

// ---------------------------------------------------------------------------
// write_kv: token i's [H_kv][d] K and V rows go to slot slot_mapping[i]; one
// thread per 16-byte chunk of an input row, a plain copy of bits into the tile
// layouts: K tiles are [d / x][16][x] (the chunk lands whole at (chunk, offset)),
// V tiles are [d][16] (the chunk's x elements land in x different columns).
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void write_kv_kernel(char* k_pool, char* v_pool,
                                                       const uint4* k_new, const uint4* v_new,
                                                       const int64_t* slot_mapping, int num_tokens,
                                                       int64_t num_slots, int num_kv_heads,
                                                       int chunks_per_row) {
  constexpr int kX = 16 / sizeof(E);  // elements per chunk
  const int chunks_per_token = num_kv_heads * chunks_per_row;
  const int64_t total = static_cast<int64_t>(num_tokens) * chunks_per_token;
  const size_t tile_bytes = static_cast<size_t>(kBlockSize) * chunks_per_row * 16;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int tok = static_cast<int>(idx / chunks_per_token);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int rem = static_cast<int>(idx % chunks_per_token);
    const int g = rem / chunks_per_row;
    const int ch = rem % chunks_per_row;
    const int64_t phys = slot / kBlockSize;
    const int o = static_cast<int>(slot % kBlockSize);
    const size_t tile = (static_cast<size_t>(phys) * num_kv_heads + g) * tile_bytes;
    *reinterpret_cast<uint4*>(k_pool + tile + (static_cast<size_t>(ch) * kBlockSize + o) * 16) = k_new[idx];
    const uint4 v = v_new[idx];
    E e[kX];
    __builtin_memcpy(e, &v, 16);
    E* vt = reinterpret_cast<E*>(v_pool + tile);
#pragma unroll
    for (int i = 0; i < kX; ++i) vt[(ch * kX + i) * kBlockSize + o] = e[i];
  }
}

// ---------------------------------------------------------------------------
// debug: the slots the decode kernels read, from the same device function
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slot_ids_kernel(const int32_t* block_tables,
                                                       int max_blocks_per_seq,
                                                       const int32_t* context_lens, int num_seqs,
                                                       int max_context_len, int num_blocks,
                                                       int64_t* slot_ids) {
  const int64_t total = static_cast<int64_t>(num_seqs) * max_context_len;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int s = static_cast<int>(idx / max_context_len);
    const int t = static_cast<int>(idx % max_context_len);
    const int L = pa_clamp_len(context_lens[s], max_context_len);
    int64_t v = -1;
    if (t < L) {
      const int32_t* row = block_tables + static_cast<size_t>(s) * max_blocks_per_seq;
      v = pa_slot(pa_physical_block(row, t / kBlockSize, num_blocks), t);
    }
    slot_ids[idx] = v;
  }
}

unsigned grid_for(int64_t n, int threads) {
  const int64_t g = (n + threads - 1) / threads;
  return static_cast<unsigned>(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case PA_F32: return launch_reduce_t<F32>(a, stream);
    case PA_F16: return launch_reduce_t<F16>(a, stream);
    default: return launch_reduce_t<BF16>(a, stream);
  }
}

hipError_t launch_fill(void* dst, size_t bytes, uint32_t pattern, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(static_cast<int64_t>(n16), 256)), dim3(256), 0,
                     stream, static_cast<uint4*>(dst), n16, pattern);
  return hipGetLastError();
}

hipError_t launch_write_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                           int32_t num_kv_heads, int32_t row_bytes, int32_t elem_bytes,
                           hipStream_t stream) {
  const int chunks_per_row = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * chunks_per_row;
  auto kernel = elem_bytes == 4 ? write_kv_kernel<uint32_t> : write_kv_kernel<uint16_t>;
  hipLaunchKernelGGL(kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     slot_mapping, num_tokens, static_cast<int64_t>(num_blocks) * kBlockSize,
                     num_kv_heads, chunks_per_row);
  return hipGetLastError();
}

hipError_t launch_slot_ids(const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           int32_t num_blocks, int64_t* slot_ids, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(num_seqs) * max_context_len;
  hipLaunchKernelGGL(slot_ids_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                     num_blocks, slot_ids);
  return hipGetLastError();
}

}  // namespace pa
