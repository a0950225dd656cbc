// Paged decode attention, vector-ALU kernel (all dtypes, head_dim 64 / 128).
//
// One workgroup of kWaves wavefronts owns (sequence s, KV head g, a chunk of
// kHeads query heads of g's group, partition p).  The partition's 16-token
// blocks are dealt round-robin to the waves.  For one block a wave reads the
// K tile and the V tile (each 16 rows x D elements, contiguous in the pool) with
// fully coalesced 16-byte loads: load i of a tile covers bytes [1024 i, 1024 i +
// 1024), so lane l holds row i * kTpi + l / kLpr and kVec consecutive columns.
// The next block's tiles are in flight while the current one is consumed.
//
// Per block and query head: logits by per-lane FMAs and a DPP sum over the kLpr
// lanes of a row, then an online-softmax update -- the running maximum and sum
// are carried while streaming, with the accumulator rescaled when the maximum
// grows (§4.2 of the ialgorithm.me page, "大模型推理加速与显存黑科技").  Each
// row of lanes keeps its own running state; rows, then waves, are merged with
// the same log-sum-exp algebra at the end, in a fixed order (no atomics, so a
// run is bit-reproducible).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <class Tr, int D, int kHeads, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(DecodeArgs a) {
  constexpr int kVec = Tr::kVec;            // elements per 16-byte load
  constexpr int kLpr = D / kVec;            // lanes that hold one token row
  constexpr int kTpi = 64 / kLpr;           // token rows per wave load
  constexpr int kNi = kBlockSize / kTpi;    // wave loads per tile
  static_assert(kLpr >= 1 && kLpr <= 64 && kTpi * kNi == kBlockSize, "tile mapping");

  __shared__ float sm_acc[kWaves][kHeads][D];
  __shared__ float sm_m[kWaves][kHeads];
  __shared__ float sm_l[kWaves][kHeads];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int part = blockIdx.x;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int chunks = group / kHeads;
  const int g = blockIdx.y / chunks;
  const int h0 = g * group + (blockIdx.y % chunks) * kHeads;
  const int s = blockIdx.z;

  const int L = pa_clamp_len(a.context_lens[s], a.max_context_len);
  const int t_lo = part * a.partition_tokens;
  const int t_hi = min(L, t_lo + a.partition_tokens);
  const int blk_lo = t_lo / kBlockSize;
  const int blk_hi = t_hi > t_lo ? (t_hi + kBlockSize - 1) / kBlockSize : blk_lo;

  const int row = lane / kLpr;
  const int col0 = (lane % kLpr) * kVec;

  // query rows, pre-multiplied by scale * log2(e) so that exp2 gives the weights
  float qv[kHeads][kVec];
  const float qs = a.scale * kLog2e;
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    const size_t off = ((static_cast<size_t>(s) * a.num_q_heads + h0 + h) * D + col0) * Tr::kBytes;
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + off);
    Tr::unpack(u, qv[h]);
#pragma unroll
    for (int e = 0; e < kVec; ++e) qv[h][e] *= qs;
  }

  float m[kHeads], l[kHeads], acc[kHeads][kVec];
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[h][e] = 0.f;
  }

  const int32_t* __restrict__ trow = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
  const char* __restrict__ kbase = static_cast<const char*>(a.k_pool);
  const char* __restrict__ vbase = static_cast<const char*>(a.v_pool);

  auto load = [&](int j, uint4 (&kr)[kNi], uint4 (&vr)[kNi]) {
    const int phys = pa_physical_block(trow, j, a.num_blocks);
    const size_t off = pa_tile_offset(phys, g, a.num_kv_heads, D) * Tr::kBytes;
    const uint4* kt = reinterpret_cast<const uint4*>(kbase + off);
    const uint4* vt = reinterpret_cast<const uint4*>(vbase + off);
#pragma unroll
    for (int i = 0; i < kNi; ++i) kr[i] = kt[i * 64 + lane];
#pragma unroll
    for (int i = 0; i < kNi; ++i) vr[i] = vt[i * 64 + lane];
  };

  auto consume = [&](int j, uint4 (&kr)[kNi], uint4 (&vr)[kNi]) {
    float sc[kNi][kHeads];
#pragma unroll
    for (int i = 0; i < kNi; ++i) {
      float kf[kVec];
      Tr::unpack(kr[i], kf);
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        float d0 = 0.f;
#pragma unroll
        for (int e = 0; e < kVec; ++e) d0 = fmaf(qv[h][e], kf[e], d0);
        sc[i][h] = group_sum<kLpr>(d0);
      }
    }
    // the last block of a range is partial: its dead rows may hold anything
    // (NaN included), so logits are selected to -inf and V rows to zero
    if ((j + 1) * kBlockSize > t_hi) {
#pragma unroll
      for (int i = 0; i < kNi; ++i) {
        if (j * kBlockSize + i * kTpi + row >= t_hi) {
#pragma unroll
          for (int h = 0; h < kHeads; ++h) sc[i][h] = -INFINITY;
          vr[i] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
    float pr[kNi][kHeads];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int i = 1; i < kNi; ++i) bm = fmaxf(bm, sc[i][h]);
      const float mn = fmaxf(m[h], bm);
      const bool dead = mn == -INFINITY;  // nothing seen yet by this row
      const float alpha = dead ? 1.f : __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < kNi; ++i) {
        pr[i][h] = dead ? 0.f : __builtin_amdgcn_exp2f(sc[i][h] - mn);
        l[h] += pr[i][h];
      }
    }
#pragma unroll
    for (int i = 0; i < kNi; ++i) {
      float vf[kVec];
      Tr::unpack(vr[i], vf);
#pragma unroll
      for (int h = 0; h < kHeads; ++h)
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[h][e] = fmaf(pr[i][h], vf[e], acc[h][e]);
    }
  };

  // two register sets: block j is consumed while block j + kWaves is loading
  uint4 ka[kNi], va[kNi], kb[kNi], vb[kNi];
  int j = blk_lo + wave;
  if (j < blk_hi) load(j, ka, va);
  while (j < blk_hi) {
    int jn = j + kWaves;
    if (jn < blk_hi) load(jn, kb, vb);
    consume(j, ka, va);
    j = jn;
    if (j >= blk_hi) break;
    jn = j + kWaves;
    if (jn < blk_hi) load(jn, ka, va);
    consume(j, kb, vb);
    j = jn;
  }

  // merge the rows of this wave
#pragma unroll
  for (int h = 0; h < kHeads; ++h) {
    const float M = across_groups_max<kLpr>(m[h]);
    const float f = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - M);
    l[h] = across_groups_sum<kLpr>(l[h] * f);
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[h][e] = across_groups_sum<kLpr>(acc[h][e] * f);
    m[h] = M;
  }
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < kHeads; ++h)
#pragma unroll
      for (int e = 0; e < kVec; ++e) sm_acc[wave][h][col0 + e] = acc[h][e];
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // merge the waves and write
  for (int idx = threadIdx.x; idx < kHeads * D; idx += kWaves * 64) {
    const int h = idx / D;
    const int c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, lse = -INFINITY;
    if (M != -INFINITY) {
      float ls = 0.f, os = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w][h] - M);
        ls = fmaf(sm_l[w][h], f, ls);
        os = fmaf(sm_acc[w][h][c], f, os);
      }
      o = os / ls;
      lse = (M + __log2f(ls)) * kLn2;
    }
    const size_t r = static_cast<size_t>(s) * a.num_q_heads + h0 + h;
    if (a.write_partials) {
      a.o_part[(r * a.num_parts + part) * D + c] = o;
      if (c == 0) a.lse_part[r * a.num_parts + part] = lse;
    } else {
      Tr::store(a.out, r * D + c, o);
    }
  }
}

template <class Tr, int D, int kHeads>
hipError_t launch_valu(const DecodeArgs& a, hipStream_t stream) {
  constexpr int kWaves = 4;
  const int chunks = (a.num_q_heads / a.num_kv_heads) / kHeads;
  dim3 grid(a.num_parts, a.num_kv_heads * chunks, a.num_seqs);
  hipLaunchKernelGGL((decode_valu_kernel<Tr, D, kHeads, kWaves>), grid, dim3(kWaves * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <class Tr, int D>
hipError_t launch_valu_heads(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  // float32 rows of 128 need twice the registers per head: at most 4 heads
  constexpr bool kWide = Tr::kBytes * D > 256;
  if constexpr (!kWide) {
    if (group % 8 == 0) return launch_valu<Tr, D, 8>(a, stream);
  }
  if (group % 4 == 0) return launch_valu<Tr, D, 4>(a, stream);
  if (group % 2 == 0) return launch_valu<Tr, D, 2>(a, stream);
  return launch_valu<Tr, D, 1>(a, stream);
}

template <class Tr>
hipError_t launch_valu_dim(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_valu_heads<Tr, 64>(a, stream)
                          : launch_valu_heads<Tr, 128>(a, stream);
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case PA_F32: return launch_valu_dim<F32>(a, stream);
    case PA_F16: return launch_valu_dim<F16>(a, stream);
    default: return launch_valu_dim<BF16>(a, stream);
  }
}

}  // namespace pa
