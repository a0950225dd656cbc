// The small kernels around decode: the log-sum-exp merge of partition
// partials, pool fill, KV append, whole-block moves and the debug slot-id
// gather.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// pa_reduce: one workgroup of 256 threads per (sequence, query head).  The
// partition results are re-weighted by their share of the softmax mass: with
// M = max lse_p, weight_p = exp(lse_p - M) / sum_q exp(lse_q - M).  This is the
// same streaming-normaliser identity that makes the online softmax exact (§4.2
// of the ialgorithm.me page).
//   1. weights: thread p < live partitions computes exp(lse_p - M) into LDS
//      (M and the sum by a fixed-order block reduction);
//   2. thread t owns 4 columns (t % (D/4)) and every G-th partition starting
//      at t / (D/4), with G = 256 / (D/4) partition groups, float4 loads (the
//      first eight of them issued before step 1, since they need no weight);
//   3. the G group sums are added in group order through LDS.
// Every sum has a fixed order, so the result is bit-reproducible.
// ---------------------------------------------------------------------------
constexpr int kReduceThreads = 256;

__device__ __forceinline__ float block_max_256(float v, float* sm) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  __syncthreads();
  return v;
}

template <class Tr, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
  constexpr int kCols4 = D / 4;                       // float4 column groups
  constexpr int kGroups = kReduceThreads / kCols4;    // partition groups
  constexpr int kPre = 8;                             // partials loaded before the weights
  extern __shared__ float sm_w[];                     // [num_parts] weights
  __shared__ float sm_red[4];
  __shared__ float4 sm_acc[kGroups][kCols4];

  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int t = threadIdx.x;
  const size_t row = static_cast<size_t>(s) * a.num_q_heads + h;
  const int c4 = t % kCols4;
  const int grp = t / kCols4;
  const float4* op = reinterpret_cast<const float4*>(a.o_part + row * a.num_parts * D) + c4;
  // The first kPre partials of this thread do not depend on the weights (every
  // partition of the workspace was written, empty ones as zeros): issue their
  // loads first so they overlap the lse loads and the max reduction.
  float4 pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int p = grp + i * kGroups;
    pre[i] = p < a.num_parts ? op[static_cast<size_t>(p) * kCols4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int L = pa_clamp_len(a.context_lens[s], a.max_context_len);
  const int nv = (L + a.partition_tokens - 1) / a.partition_tokens;  // live partitions
  const float* lse = a.lse_part + row * a.num_parts;

  float mx = -INFINITY;
  for (int p = t; p < nv; p += kReduceThreads) mx = fmaxf(mx, lse[p]);
  const float M = block_max_256(mx, sm_red);
  if (M == -INFINITY) {  // empty context: zero row (block-uniform branch)
    for (int c = t; c < D; c += kReduceThreads) Tr::store(a.out, row * D + c, 0.f);
    return;
  }
  for (int p = t; p < nv; p += kReduceThreads) sm_w[p] = __expf(lse[p] - M);
  __syncthreads();

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int p = grp + i * kGroups;
    if (p < nv) {
      const float w = sm_w[p];
      acc.x = fmaf(w, pre[i].x, acc.x);
      acc.y = fmaf(w, pre[i].y, acc.y);
      acc.z = fmaf(w, pre[i].z, acc.z);
      acc.w = fmaf(w, pre[i].w, acc.w);
    }
  }
  for (int p = grp + kPre * kGroups; p < nv; p += kGroups) {
    const float w = sm_w[p];
    const float4 v = op[static_cast<size_t>(p) * kCols4];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  sm_acc[grp][c4] = acc;
  __syncthreads();
  if (t < kCols4) {
    float wsum = 0.f;
    for (int p = 0; p < nv; ++p) wsum += sm_w[p];
    const float inv = 1.f / wsum;
    float4 o = sm_acc[0][t];
#pragma unroll
    for (int g = 1; g < kGroups; ++g) {
      o.x += sm_acc[g][t].x;
      o.y += sm_acc[g][t].y;
      o.z += sm_acc[g][t].z;
      o.w += sm_acc[g][t].w;
    }
    const size_t base = row * D + 4 * t;
    Tr::store(a.out, base + 0, o.x * inv);
    Tr::store(a.out, base + 1, o.y * inv);
    Tr::store(a.out, base + 2, o.z * inv);
    Tr::store(a.out, base + 3, o.w * inv);
  }
}

template <class Tr>
hipError_t launch_reduce_t(const ReduceArgs& a, hipStream_t stream) {
  dim3 grid(a.num_q_heads, a.num_seqs);
  const size_t lds = static_cast<size_t>(a.num_parts) * sizeof(float);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((reduce_kernel<Tr, 64>), grid, dim3(kReduceThreads), lds, stream, a);
  else
    hipLaunchKernelGGL((reduce_kernel<Tr, 128>), grid, dim3(kReduceThreads), lds, stream, a);
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
// layouts of bs-token blocks: K tiles are [d / x][bs][x] (the chunk lands whole
// at (chunk, offset)), V tiles are [d][bs] (the chunk's x elements land in x
// different columns).
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void write_kv_kernel(char* k_pool, char* v_pool,
                                                       const uint4* k_new, const uint4* v_new,
                                                       const int64_t* slot_mapping, int num_tokens,
                                                       int64_t num_slots, int bs, int num_kv_heads,
                                                       int chunks_per_row) {
  constexpr int kX = 16 / sizeof(E);  // elements per chunk
  const int chunks_per_token = num_kv_heads * chunks_per_row;
  const int64_t total = static_cast<int64_t>(num_tokens) * chunks_per_token;
  const size_t tile_bytes = static_cast<size_t>(bs) * chunks_per_row * 16;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int tok = static_cast<int>(idx / chunks_per_token);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int rem = static_cast<int>(idx % chunks_per_token);
    const int g = rem / chunks_per_row;
    const int ch = rem % chunks_per_row;
    const int64_t phys = slot / bs;
    const int o = static_cast<int>(slot % bs);
    const size_t tile = (static_cast<size_t>(phys) * num_kv_heads + g) * tile_bytes;
    *reinterpret_cast<uint4*>(k_pool + tile + (static_cast<size_t>(ch) * bs + o) * 16) = k_new[idx];
    const uint4 v = v_new[idx];
    E e[kX];
    __builtin_memcpy(e, &v, 16);
    E* vt = reinterpret_cast<E*>(v_pool + tile);
#pragma unroll
    for (int i = 0; i < kX; ++i) vt[(ch * kX + i) * bs + o] = e[i];
  }
}

// ---------------------------------------------------------------------------
// write_kv_k8: as write_kv, with each key element quantised to int8 by its
// channel's scale: code = clamp(rint(k / scale), -127, 127), the quotient an
// IEEE float32 division rounded to nearest and rint rounding ties to even.
// One thread per 16 channels of one token and KV head: two 16-byte loads of
// the 16-bit key row, one 16-byte store of codes into the int8 tile
// ([d / 16][bs][16]); the 16 value elements land in 16 columns of the V tile.
// ---------------------------------------------------------------------------
template <class Tr, typename E>
__global__ __launch_bounds__(256) void write_kv_k8_kernel(char* k_pool, char* v_pool,
                                                          const float* k_scale,
                                                          const uint4* k_new, const uint4* v_new,
                                                          const int64_t* slot_mapping,
                                                          int num_tokens, int64_t num_slots, int bs,
                                                          int num_kv_heads, int head_dim) {
  const int groups = head_dim / 16;  // 16-channel groups per row
  const int per_token = num_kv_heads * groups;
  const int64_t total = static_cast<int64_t>(num_tokens) * per_token;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int tok = static_cast<int>(idx / per_token);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int rem = static_cast<int>(idx % per_token);
    const int g = rem / groups;
    const int cg = rem % groups;
    const int64_t phys = slot / bs;
    const int o = static_cast<int>(slot % bs);
    const size_t tile = (static_cast<size_t>(phys) * num_kv_heads + g) * bs * head_dim;
    const size_t row = (static_cast<size_t>(tok) * num_kv_heads + g) * head_dim + 16 * cg;  // elements
    float kf[16];
    Tr::unpack(k_new[row / 8], kf);
    Tr::unpack(k_new[row / 8 + 1], kf + 8);
    const float* sc = k_scale + static_cast<size_t>(g) * head_dim + 16 * cg;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float c = __builtin_rintf(__fdiv_rn(kf[e], sc[e]));
      c = fminf(fmaxf(c, -127.f), 127.f);
      const uint32_t b = static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xffu;
      w[e / 4] |= b << (8 * (e % 4));
    }
    *reinterpret_cast<uint4*>(k_pool + tile + (static_cast<size_t>(cg) * bs + o) * 16) =
        make_uint4(w[0], w[1], w[2], w[3]);
    E ve[16];
    __builtin_memcpy(ve, &v_new[row / 8], 16);
    __builtin_memcpy(ve + 8, &v_new[row / 8 + 1], 16);
    E* vt = reinterpret_cast<E*>(v_pool) + tile;
#pragma unroll
    for (int e = 0; e < 16; ++e) vt[(16 * cg + e) * bs + o] = ve[e];
  }
}

// ---------------------------------------------------------------------------
// whole-block moves (copy-on-write copies, swap gather / scatter).  Pair p
// moves block src(p) of the source K and V buffers to block dst(p) of the
// destination ones, where src(p) = src_ids[p * src_stride] (or p when src_ids
// is null) and likewise for dst.  A block is block_bytes of contiguous tiles
// (every KV head; K and V blocks may differ in size).  Pairs with an id outside
// its buffer's limit are skipped, and
// so are src == dst pairs when skip_equal is set (a copy inside one pool).
// blockIdx.z selects K (0) or V (1); pairs are strided over blockIdx.y.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_move_kernel(const uint4* src_k, const uint4* src_v,
                                                         uint4* dst_k, uint4* dst_v,
                                                         const int32_t* src_ids, int src_stride,
                                                         int src_limit, const int32_t* dst_ids,
                                                         int dst_stride, int dst_limit,
                                                         int num_pairs, size_t k_block16,
                                                         size_t v_block16, bool skip_equal) {
  const uint4* src = blockIdx.z == 0 ? src_k : src_v;
  uint4* dst = blockIdx.z == 0 ? dst_k : dst_v;
  const size_t block16 = blockIdx.z == 0 ? k_block16 : v_block16;
  for (int p = blockIdx.y; p < num_pairs; p += gridDim.y) {
    const int sb = src_ids ? src_ids[static_cast<size_t>(p) * src_stride] : p;
    const int db = dst_ids ? dst_ids[static_cast<size_t>(p) * dst_stride] : p;
    if (sb < 0 || sb >= src_limit || db < 0 || db >= dst_limit) continue;
    if (skip_equal && sb == db) continue;
    const uint4* s = src + static_cast<size_t>(sb) * block16;
    uint4* d = dst + static_cast<size_t>(db) * block16;
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < block16;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
      d[i] = s[i];
  }
}

// ---------------------------------------------------------------------------
// debug: the slots the decode kernels read, from the same device function
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slot_ids_kernel(const int32_t* block_tables,
                                                       int max_blocks_per_seq,
                                                       const int32_t* context_lens, int num_seqs,
                                                       int max_context_len, int num_blocks, int bs,
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
      v = pa_slot(pa_physical_block(row, t / bs, num_blocks), t, bs);
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
                           int32_t block_size, int32_t num_kv_heads, int32_t row_bytes,
                           int32_t elem_bytes, hipStream_t stream) {
  const int chunks_per_row = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * chunks_per_row;
  auto kernel = elem_bytes == 4 ? write_kv_kernel<uint32_t> : write_kv_kernel<uint16_t>;
  hipLaunchKernelGGL(kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     slot_mapping, num_tokens, static_cast<int64_t>(num_blocks) * block_size,
                     block_size, num_kv_heads, chunks_per_row);
  return hipGetLastError();
}

hipError_t launch_write_kv_k8(void* k_pool, void* v_pool, const float* k_scale, const void* k_new,
                              const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim / 16);
  auto kernel = dtype == PA_K8_F16 ? write_kv_k8_kernel<F16, uint16_t>
                                   : write_kv_k8_kernel<BF16, uint16_t>;
  hipLaunchKernelGGL(kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), k_scale,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     slot_mapping, num_tokens, static_cast<int64_t>(num_blocks) * block_size,
                     block_size, num_kv_heads, head_dim);
  return hipGetLastError();
}

hipError_t launch_block_move(const BlockMoveArgs& a, hipStream_t stream) {
  const size_t k16 = a.k_block_bytes / 16, v16 = a.v_block_bytes / 16;
  const size_t block16 = k16 > v16 ? k16 : v16;
  const int64_t xg = static_cast<int64_t>((block16 + 255) / 256);
  const unsigned gx = static_cast<unsigned>(xg < 1 ? 1 : (xg > 64 ? 64 : xg));
  const unsigned gy = static_cast<unsigned>(a.num_pairs < 1 ? 1 : (a.num_pairs > 65535 ? 65535 : a.num_pairs));
  hipLaunchKernelGGL(block_move_kernel, dim3(gx, gy, 2), dim3(256), 0, stream,
                     static_cast<const uint4*>(a.src_k), static_cast<const uint4*>(a.src_v),
                     static_cast<uint4*>(a.dst_k), static_cast<uint4*>(a.dst_v), a.src_ids,
                     a.src_stride, a.src_limit, a.dst_ids, a.dst_stride, a.dst_limit, a.num_pairs,
                     k16, v16, a.skip_equal);
  return hipGetLastError();
}

hipError_t launch_slot_ids(const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           int32_t num_blocks, int32_t block_size, int64_t* slot_ids,
                           hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(num_seqs) * max_context_len;
  hipLaunchKernelGGL(slot_ids_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                     num_blocks, block_size, slot_ids);
  return hipGetLastError();
}

}  // namespace pa
