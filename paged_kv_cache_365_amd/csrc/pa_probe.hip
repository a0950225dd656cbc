// Read-only probes that give the decode kernel's roofline its achievable
// context: how fast this GPU streams plain contiguous memory, and how fast it
// streams the K/V tiles a decode call reads, in the decode kernel's order and
// with its loads, when nothing is computed on them.  Decode is bound by these
// reads (the pages put the cost of attention in moving K/V between HBM and the
// chip: §4.1 of the ialgorithm.me page, §3.1 of the blog.tanteng.space page).
//
// Each probe folds what it reads into one 32-bit XOR per wavefront, so the
// loads cannot be dropped, and writes those words to a small sink.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }
__device__ __forceinline__ uint32_t fold(u32x2 v) { return v.x ^ v.y; }

// XOR over the 64 lanes; lane 0 of each wave writes its word.
__device__ __forceinline__ void sink_wave(uint32_t acc, uint32_t* sink, size_t index) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) sink[index] = acc;
}

// Contiguous streaming read: each wavefront reads whole 4 KiB runs (four
// 1 KiB loads of 16 bytes per lane, the decode tile's size), runs dealt to the
// wavefronts round-robin, two runs in flight; the last partial run is read by
// the first workgroup.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t wave = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const size_t waves = static_cast<size_t>(gridDim.x) * 4;
  const size_t runs = n16 / 256;
  uint32_t acc = 0;
  auto run = [&](size_t k) {
    const u32x4* p = src + k * 256 + lane;
    return fold(__builtin_nontemporal_load(p)) ^ fold(__builtin_nontemporal_load(p + 64)) ^
           fold(__builtin_nontemporal_load(p + 128)) ^ fold(__builtin_nontemporal_load(p + 192));
  };
  size_t k = wave;
  for (; k + waves < runs; k += 2 * waves) acc ^= run(k) ^ run(k + waves);
  if (k < runs) acc ^= run(k);
  if (blockIdx.x == 0)
    for (size_t i = runs * 256 + threadIdx.x; i < n16; i += 256) acc ^= fold(__builtin_nontemporal_load(src + i));
  sink_wave(acc, sink, static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6));
}

// The decode kernel's tile reads for 16-bit pools in 16-token blocks: one
// workgroup of 8 waves per (sequence, KV head), wave w reads the 16-token steps
// w, w + 8, ... through the block table, two steps in flight; per step every
// lane reads its 16-byte K chunks (tile + 1 KiB * j + 16 * lane) and its
// 8-byte V runs (4 tokens of one column), the loads of the decode kernel.
template <int D>
__global__ __launch_bounds__(512) void probe_tiles_kernel(const char* __restrict__ k_pool,
                                                          const char* __restrict__ v_pool,
                                                          const int32_t* __restrict__ block_tables,
                                                          const int32_t* __restrict__ context_lens,
                                                          int32_t max_blocks_per_seq,
                                                          int32_t num_kv_heads, int32_t num_blocks,
                                                          int32_t max_context_len,
                                                          uint32_t* __restrict__ sink) {
  constexpr int kK = D / 32;  // 16-byte K loads per lane per tile (16 tokens x D x 2 bytes)
  constexpr int kV = D / 16;  // 8-byte V loads per lane per tile
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int qg = lane >> 4;
  const int wave = wave_id();
  const int g = blockIdx.x % num_kv_heads;
  const int s = blockIdx.x / num_kv_heads;
  const int L = pa_clamp_len(context_lens[s], max_context_len);
  const int steps = (L + kStep - 1) / kStep;
  const int32_t* trow = block_tables + static_cast<size_t>(s) * max_blocks_per_seq;
  uint32_t acc = 0;
  auto step = [&](int k) {
    const size_t tile = pa_tile_offset(pa_physical_block(trow, k, num_blocks), g, num_kv_heads, D,
                                       16) * 2;
    const u32x4* kt = reinterpret_cast<const u32x4*>(k_pool + tile);
    const u32x2* vt = reinterpret_cast<const u32x2*>(v_pool + tile);
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < kK; ++j) x ^= fold(__builtin_nontemporal_load(kt + 64 * j + lane));
#pragma unroll
    for (int cb = 0; cb < kV; ++cb) x ^= fold(__builtin_nontemporal_load(vt + (16 * cb + r) * 4 + qg));
    return x;
  };
  int k = wave;
  for (; k + 8 < steps; k += 16) acc ^= step(k) ^ step(k + 8);
  if (k < steps) acc ^= step(k);
  sink_wave(acc, sink, static_cast<size_t>(blockIdx.x) * 8 + wave);
}

}  // namespace
}  // namespace pa

extern "C" {

pa_status pa_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_words,
                        hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || sink_words < 4 || sink_words % 4 != 0)
    return PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return PA_ERR_MISALIGNED;
  hipLaunchKernelGGL(pa::probe_read_kernel, dim3(sink_words / 4), dim3(256), 0, stream,
                     static_cast<const pa::u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_probe_read_tiles(const pa_pool_desc* pool, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, uint32_t* sink, int32_t sink_words,
                              hipStream_t stream) {
  if (!pool || !k_pool || !v_pool || !block_tables || !context_lens || !sink)
    return PA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || pool->num_blocks <= 0 ||
      pool->num_kv_heads <= 0)
    return PA_ERR_INVALID_ARG;
  if ((pool->dtype != PA_F16 && pool->dtype != PA_BF16) || pool->block_size != 16 ||
      (pool->head_dim != 64 && pool->head_dim != 128))
    return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * 16)
    return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_seqs) * pool->num_kv_heads > INT32_MAX / 8) return PA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(sink_words) < static_cast<int64_t>(num_seqs) * pool->num_kv_heads * 8)
    return PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(k_pool) % 16 != 0 || reinterpret_cast<uintptr_t>(v_pool) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(block_tables) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(context_lens) % 4 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return PA_ERR_MISALIGNED;
  const dim3 grid(num_seqs * pool->num_kv_heads);
  if (pool->head_dim == 128) {
    hipLaunchKernelGGL(pa::probe_tiles_kernel<128>, grid, dim3(512), 0, stream,
                       static_cast<const char*>(k_pool), static_cast<const char*>(v_pool),
                       block_tables, context_lens, max_blocks_per_seq, pool->num_kv_heads,
                       pool->num_blocks, max_context_len, sink);
  } else {
    hipLaunchKernelGGL(pa::probe_tiles_kernel<64>, grid, dim3(512), 0, stream,
                       static_cast<const char*>(k_pool), static_cast<const char*>(v_pool),
                       block_tables, context_lens, max_blocks_per_seq, pool->num_kv_heads,
                       pool->num_blocks, max_context_len, sink);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
