// The small kernels around decode: the log-sum-exp merge of partition
// partials, pool fill, KV append, whole-block moves and the debug slot-id
// gather.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// pa_reduce: one wavefront per (row, column slice), four per workgroup.  The
// partition results are re-weighted by their share of the softmax mass: with
// M = max lse_p, weight_p = exp(lse_p - M) / sum_q exp(lse_q - M).  This is the
// same streaming-normaliser identity that makes the online softmax exact (§4.2
// of the ialgorithm.me page).
//   lane l = C g + c (C = 64 / kGroups float4 columns, a slice of 4 C columns):
//   float4 column c of the slice, partitions g, g + kGroups, ...;
//   1. the first kPre partials of the lane and their lse are loaded before
//      anything else (they need no weight), the maximum M is a lane-strided
//      scan of the live lse values and a butterfly over the wavefront;
//   2. each lane weights and sums its partitions and their weights;
//   3. a butterfly over the partition groups adds the group sums; the lanes of
//      group 0 normalise and store.
// kGroups = 8 (32-column slices) for many partitions; with at most 4 or 2
// partitions per row, 4 or 2 groups and 64- or 128-column slices, so a row
// takes fewer wavefronts and fewer lanes idle (shared-prefix batch, 2
// partitions per row: 16384 -> 4096 wavefronts).
// No LDS and no barrier.  Every sum has a fixed order and the butterfly gives
// every lane the same bits, so the result is reproducible run to run.
// ---------------------------------------------------------------------------
constexpr int kReduceWaves = 4;    // wavefronts per workgroup

template <class Tr, int D, int kGroups>
__global__ __launch_bounds__(64 * kReduceWaves) void reduce_kernel(ReduceArgs a) {
  constexpr int kCols = 64 / kGroups;      // float4 columns per slice
  constexpr int kSliceCols = 4 * kCols;    // output columns per wavefront
  static_assert(kSliceCols <= D, "a slice lies inside one row");
  constexpr int kSlices = D / kSliceCols;
  constexpr int kPre = kGroups == 8 ? 8 : 1;  // partials per lane loaded up front
  const int lane = threadIdx.x & 63;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kReduceWaves + (threadIdx.x >> 6);
  if (unit >= static_cast<int64_t>(a.num_seqs) * a.num_q_heads * kSlices) return;
  const int64_t row = unit / kSlices;
  const int slice = static_cast<int>(unit % kSlices);
  const int s = static_cast<int>(row / a.num_q_heads);
  const int c4 = lane % kCols;
  const int grp = lane / kCols;
  const int col = slice * kSliceCols + 4 * c4;
  const float* lse = a.lse_part + row * a.num_parts;
  const float* op = a.o_part + row * a.num_parts * D + col;

  float4 pre[kPre];
  float lpre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int p = grp + i * kGroups;
    if (p < a.num_parts) {
      pre[i] = *reinterpret_cast<const float4*>(op + static_cast<size_t>(p) * D);
      lpre[i] = lse[p];
    } else {
      pre[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      lpre[i] = -INFINITY;
    }
  }
  const int L = pa_clamp_len(a.context_lens[s], a.max_context_len);
  const int nv = (L + a.partition_tokens - 1) / a.partition_tokens;  // live partitions

  float M = -INFINITY;
#pragma unroll 4
  for (int p = lane; p < nv; p += 64) M = fmaxf(M, lse[p]);
  M = across_groups_max<1>(M);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (M != -INFINITY) {  // wavefront-uniform: an empty context stores a zero row
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      if (grp + i * kGroups < nv) {
        const float w = __expf(lpre[i] - M);
        acc.x = fmaf(w, pre[i].x, acc.x);
        acc.y = fmaf(w, pre[i].y, acc.y);
        acc.z = fmaf(w, pre[i].z, acc.z);
        acc.w = fmaf(w, pre[i].w, acc.w);
        wsum += w;
      }
    }
#pragma unroll 4
    for (int p = grp + kPre * kGroups; p < nv; p += kGroups) {
      const float w = __expf(lse[p] - M);
      const float4 v = *reinterpret_cast<const float4*>(op + static_cast<size_t>(p) * D);
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
      wsum += w;
    }
    acc.x = across_groups_sum<kCols>(acc.x);
    acc.y = across_groups_sum<kCols>(acc.y);
    acc.z = across_groups_sum<kCols>(acc.z);
    acc.w = across_groups_sum<kCols>(acc.w);
    wsum = across_groups_sum<kCols>(wsum);
    const float inv = 1.f / wsum;
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;
  }
  if (grp == 0) {
    const size_t base = static_cast<size_t>(row) * D + col;
    Tr::store(a.out, base + 0, acc.x);
    Tr::store(a.out, base + 1, acc.y);
    Tr::store(a.out, base + 2, acc.z);
    Tr::store(a.out, base + 3, acc.w);
  }
}

template <class Tr, int D, int kGroups>
hipError_t launch_reduce_g(const ReduceArgs& a, hipStream_t stream) {
  constexpr int kSlices = D / (256 / kGroups);
  const int64_t units = static_cast<int64_t>(a.num_seqs) * a.num_q_heads * kSlices;
  const dim3 grid(static_cast<uint32_t>((units + kReduceWaves - 1) / kReduceWaves));
  hipLaunchKernelGGL((reduce_kernel<Tr, D, kGroups>), grid, dim3(64 * kReduceWaves), 0, stream, a);
  return hipGetLastError();
}

template <class Tr>
hipError_t launch_reduce_t(const ReduceArgs& a, hipStream_t stream) {
  if (a.head_dim == 64)
    return a.num_parts <= 4 ? launch_reduce_g<Tr, 64, 4>(a, stream)
                            : launch_reduce_g<Tr, 64, 8>(a, stream);
  if (a.num_parts <= 2) return launch_reduce_g<Tr, 128, 2>(a, stream);
  return a.num_parts <= 4 ? launch_reduce_g<Tr, 128, 4>(a, stream)
                          : launch_reduce_g<Tr, 128, 8>(a, stream);
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

// write_kv_k2: as write_kv, with each key element quantised to a 2-bit code
// by its channel's step s and zero point z: u = (k - z) / s in float32 (IEEE
// subtraction and division), code = rint(min(max(u, 0), 3)) (fminf/fmaxf drop a
// NaN).  One thread per (token, KV head, key word): word (q, w) of a token holds
// channels 32 j + 8 q + e for j = 2w + h, h = 0, 1, e = 0..7, the code of
// channel 32 j + 8 q + 2 i + p at bit 2 (4 h + i) + 16 p -- two contiguous runs of
// 8 channels of the new row.  A thread also copies the V elements of those 16
// channels.
template <class Tr, class E>
__global__ __launch_bounds__(256) void write_kv_k2_kernel(char* k_pool, char* v_pool,
                                                          const float* k_scale, const float* k_zero,
                                                          const uint4* k_new, const uint4* v_new,
                                                          const int64_t* slot_mapping,
                                                          int num_tokens, int64_t num_slots, int bs,
                                                          int num_kv_heads, int head_dim) {
  const int cols = head_dim / 64;     // words per (group, token)
  const int words = 4 * cols;         // words per token and KV head
  const int per_token = num_kv_heads * words;
  const int64_t total = static_cast<int64_t>(num_tokens) * per_token;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int tok = static_cast<int>(idx / per_token);
    const int64_t slot = slot_mapping[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int rem = static_cast<int>(idx % per_token);
    const int g = rem / words;
    const int q = (rem % words) / cols;
    const int w = rem % cols;
    const int64_t phys = slot / bs;
    const int o = static_cast<int>(slot % bs);
    const size_t tile = (static_cast<size_t>(phys) * num_kv_heads + g) * bs * head_dim;  // elements
    const size_t row = (static_cast<size_t>(tok) * num_kv_heads + g) * head_dim;          // elements
    uint32_t word = 0u;
    E* vt = reinterpret_cast<E*>(v_pool) + tile;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c0 = 32 * (2 * w + h) + 8 * q;  // first of the 8 channels
      float kf[8];
      Tr::unpack(k_new[(row + c0) / 8], kf);
      const float* sc = k_scale + static_cast<size_t>(g) * head_dim + c0;
      const float* zp = k_zero + static_cast<size_t>(g) * head_dim + c0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float u = __fdiv_rn(kf[e] - zp[e], sc[e]);
        u = __builtin_rintf(fminf(fmaxf(u, 0.f), 3.f));
        word |= static_cast<uint32_t>(u) << (2 * (4 * h + e / 2) + 16 * (e % 2));
      }
      E ve[8];
      __builtin_memcpy(ve, &v_new[(row + c0) / 8], 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(c0 + e) * bs + o] = ve[e];
    }
    // word [q][o][w] of the tile: bs * head_dim / 16 words per tile
    reinterpret_cast<uint32_t*>(k_pool)[tile / 16 + (static_cast<size_t>(q) * bs + o) * cols + w] = word;
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

hipError_t launch_write_kv_k2(void* k_pool, void* v_pool, const float* k_scale, const float* k_zero,
                              const void* k_new, const void* v_new, const int64_t* slot_mapping,
                              int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                              hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim / 16);
  auto kernel = dtype == PA_K2_F16 ? write_kv_k2_kernel<F16, uint16_t>
                                   : write_kv_k2_kernel<BF16, uint16_t>;
  hipLaunchKernelGGL(kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), k_scale, k_zero,
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
