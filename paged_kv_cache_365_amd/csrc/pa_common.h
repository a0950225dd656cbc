// Device-side helpers shared by the paged decode-attention kernels (gfx950).
//
// Element types are carried as raw bits; every 16-byte load brings VEC
// elements to a lane and is widened to float32 here.  Block-table arithmetic
// lives in exactly one place (pa_clamp_block / pa_slot / pa_tile_offset) so
// that the debug slot-id kernel and the decode kernels compute the same
// addresses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

constexpr int kBlockSize = 16;  // tokens per physical block by default (8 is also built)
constexpr int kStep = 16;       // tokens per matrix-core step of the decode kernel
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kVec = 4;  // elements per 16-byte load
  static __device__ __forceinline__ void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ void store(void* base, size_t idx, float v) {
    static_cast<float*>(base)[idx] = v;
  }
};

struct F16 {
  static constexpr int kBytes = 2;
  static constexpr int kVec = 8;
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ void unpack(const uint4& u, float* f) {
    h8 h = __builtin_bit_cast(h8, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<float>(h[e]);
  }
  static __device__ __forceinline__ void store(void* base, size_t idx, float v) {
    static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(v);  // round to nearest even
  }
};

struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kVec = 8;
  // bfloat16 is the high half of a float32: widening is a shift or a mask
  static __device__ __forceinline__ void unpack(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(void* base, size_t idx, float v) {
    static_cast<__bf16*>(base)[idx] = static_cast<__bf16>(v);  // round to nearest even
  }
};

// ---------------------------------------------------------------------------
// block-table arithmetic (the only copy)
// ---------------------------------------------------------------------------
// Physical block of logical block `logical` of a table row, clamped into the
// pool so that a corrupt table cannot address memory outside it.
__device__ __forceinline__ int pa_clamp_block(int b, int num_blocks) {
  b = b < 0 ? 0 : b;
  return b >= num_blocks ? num_blocks - 1 : b;
}
__device__ __forceinline__ int pa_physical_block(const int32_t* __restrict__ table_row,
                                                 int logical, int num_blocks) {
  return pa_clamp_block(table_row[logical], num_blocks);
}
// The same for a wave-uniform logical index, read through the scalar cache
// (the constant address space: tables are never written while a kernel runs),
// so that waiting for the id counts scalar loads only and leaves the vector
// loads of K/V tiles in flight.
__device__ __forceinline__ int pa_physical_block_uniform(const int32_t* __restrict__ table_row,
                                                         int logical, int num_blocks) {
  typedef const __attribute__((address_space(4))) int32_t ScalarI32;
  return pa_clamp_block(((ScalarI32*)table_row)[__builtin_amdgcn_readfirstlane(logical)],
                        num_blocks);
}

// Slot of token t held by physical block `physical` of a pool of bs-token blocks.
__device__ __forceinline__ int64_t pa_slot(int physical, int t, int bs) {
  return static_cast<int64_t>(physical) * bs + (t % bs);
}

// Element offset of tile (physical block, kv head) in a [blocks][H_kv][bs][D] pool.
__device__ __forceinline__ size_t pa_tile_offset(int physical, int kv_head, int num_kv_heads,
                                                 int head_dim, int bs) {
  return (static_cast<size_t>(physical) * num_kv_heads + kv_head) * bs * head_dim;
}

__device__ __forceinline__ int pa_clamp_len(int len, int max_len) {
  return len < 0 ? 0 : (len > max_len ? max_len : len);
}

// ---------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------
// Reduction across the groups of kWidth lanes (lanes with equal lane % kWidth).
template <int kWidth>
__device__ __forceinline__ float across_groups_max(float v) {
#pragma unroll
  for (int off = kWidth; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
template <int kWidth>
__device__ __forceinline__ float across_groups_sum(float v) {
#pragma unroll
  for (int off = kWidth; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

}  // namespace pa
