// Paged decode attention on the matrix cores (gfx950), all element types.
//
// Rows.  A query row is one (query token, query head) pair.  Decode has one
// query token per sequence; the verify step of speculative decoding has T
// draft tokens, the last T tokens of the context, and draft token i sees the
// tokens [0, L - T + 1 + i) only (causal inside the draft).  The T * G rows of a
// sequence that share KV head g (G = query heads per KV head) read the same K/V
// tiles, so they are computed together: 16 rows per matrix-core chunk, kChunks
// chunks per workgroup (two at most), and each tile is loaded once for all of
// them.  With 16-bit keys, more than 32 rows go to workgroups of 64 whose four
// waves hold one chunk each and share every tile through LDS (kLds).  Rows
// beyond one workgroup go to sibling workgroups placed on one XCD, which read
// the tiles through that XCD's L2 (see unit_of).
//
// Work unit.  A workgroup of kWaves wavefronts owns (sequence s, KV head g, up
// to 16 * kChunks of g's rows, partition p).  The partition's 16-token steps
// are dealt round-robin to the waves; every wave streams its steps through
// registers, keeping the next step's K and V in flight while the current one
// is consumed, and carries its own online-softmax state per row.  The waves
// are merged at the end through LDS with the log-sum-exp algebra, in a fixed
// order (no atomics: runs are bit-reproducible).  In split mode over many
// partitions (kWavePart) each wave owns a whole partition instead and writes
// its partial itself.
//
// A step is 16 tokens: one 16-token block, or two 8-token blocks (kBS = 8;
// lanes r < 8 then read the first block's tile, r >= 8 the second's, see load).
// Per step, everything is two small matrix products whose operands come
// straight from the loads (lane l: r = l % 16, q = l / 16):
//
//   logits  S^T[token][row] = K[token][:] . Q[row][:]          (16 x 16 x d)
//           A = K tile: the pool stores K chunk-major ([d/x][16][x], x elements
//               per 16 bytes), so load j of a tile is the contiguous 1 KiB
//               tile[64 j + lane] = chunk 4j + q of token r: exactly lane l's
//               A operand of step j.
//           B = Q: lane l holds chunk 4j + q of query row r of the chunk (zero
//               rows pad the chunk to 16).
//           out: lane l holds the logits of tokens 4q .. 4q+3 for row r.
//   P.V     O^T[col][row] += V^T[col][token] . P^T[token][row]   (16 x 16 x 16 per 16 columns)
//           A = V tile: the pool stores V head-dim-major ([d][16]), so lane l's
//               operand (tokens 4q .. 4q+3 of column 16 cb + r) is one
//               contiguous 4-element load, and the 64 lanes read 64 * 4
//               contiguous elements.
//           B = P: lane l already holds the weights of tokens 4q .. 4q+3 for
//               row r -- the logits' own output layout -- so P never moves.
//           out: lane l holds O[row r][16 cb + 4q .. 16 cb + 4q + 3].
//   The LDS-ring workgroups (kLds) take two steps per pass: both steps'
//   logits, one softmax update for their 32 tokens, and P.V as one
//   16 x 16 x 32 product per 16 columns, whose contraction index runs over
//   the lane's 4 tokens of the first step and then of the second (pv2) -- half
//   the matrix-core instructions of two 16 x 16 x 16 products, and half the
//   barriers and softmax reductions.
//
// Int8 keys (MmaK8) feed the same logits product with f16 operands: the codes
// convert exactly and the per-channel scales ride on the query (see MmaK8).
// 2-bit keys (MmaK2) do the same with one small load per tile; their zero
// points become one logit offset per row (see MmaK2).
//
// Online softmax (§4.2 of the ialgorithm.me page: the normaliser is updated
// while streaming, exactly): the running maximum m of each row is shared by
// the four lanes holding that row (two lane-swap max steps per step).  m is
// only raised when a step's maximum exceeds it by more than kSlack (log2
// units); until then weights up to 2^kSlack are accumulated as they are.  The
// result is the same algebra (every partial sum uses one common reference), and
// the rescale of the accumulators becomes rare.  Weights are rounded to the KV
// element type for the matrix product and the running sum adds exactly the
// rounded values, so out is a true convex combination of V rows.
//
// Partial blocks: the token slots past the context end of a block may hold
// anything (NaN included); their logits are selected to -inf and their V
// elements to 0 before any arithmetic touches them.  Draft rows mask the
// tokens past their own limit the same way (those V elements are real values
// and meet weight 0).  A row that has seen no token keeps m = -inf and
// contributes nothing.
#include <type_traits>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_units.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kSlack = 8.0f;  // log2 headroom before the running maximum is raised

// Load-ring depth and cache policy (compile-time; the defaults are the
// measured best on MI355X).  Waves per workgroup are chosen per call.
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 2  // 16-token steps per wave in the load ring
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1  // streaming (non-temporal) hint on 1: K and V, 2: K, 3: V loads
#endif
constexpr int kDepth = PA_DECODE_DEPTH;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <class T>
struct NativeVec;
template <>
struct NativeVec<uint4> {
  using type = u32x4;
};
template <>
struct NativeVec<uint2> {
  using type = u32x2;
};
template <>
struct NativeVec<uint32_t> {
  using type = uint32_t;
};

// Load with or without the non-temporal hint.  K and V are each read once per
// call (shared-prefix blocks aside), so the streaming policy keeps them from
// displacing what the caches are better used for.
template <bool kStream, class T>
__device__ __forceinline__ T load16(const T* p) {
  if constexpr (kStream) {
    using N = typename NativeVec<T>::type;
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const N*>(p)));
  } else {
    return *p;
  }
}

// ---------------------------------------------------------------------------
// element-type specific operand handling
// ---------------------------------------------------------------------------
struct MmaBF16 {
  static constexpr int kKBytes = 2;  // bytes per K element
  static constexpr int kKBits = 16;  // bits per K element
  using KLoad = uint4;               // one lane's share of a K load
  static constexpr int kVBytes = 2;  // bytes per V (and q, out) element
  static constexpr int kQOps = 1;    // q operands per 16-byte K load
  using VLoad = uint2;  // 4 tokens of one V column
  using POp = uint2;    // 4 weights
  // one 16-byte chunk per lane = one 16x16x32 step
  static __device__ __forceinline__ f32x4 qk(const uint4& k, const uint4* q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q[0]), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(const VLoad& v, const POp& p, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v),
                                                     __builtin_bit_cast(s16x4, p), c, 0, 0, 0);
  }
  // round the weights (nearest even) and return the sum of the rounded values
  static __device__ __forceinline__ POp pack(const float (&p)[4], float& sum) {
    const bf16x2 a = {static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1])};
    const bf16x2 b = {static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
    const uint32_t ua = __builtin_bit_cast(uint32_t, a);
    const uint32_t ub = __builtin_bit_cast(uint32_t, b);
    // the running sum takes both rounded weights of a pair in one dot product
    // with (1, 1): the products are exact, and one instruction replaces the
    // widening and adding of each half
    const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    sum = __builtin_amdgcn_fdot2_f32_bf16(a, one, sum, false);
    sum = __builtin_amdgcn_fdot2_f32_bf16(b, one, sum, false);
    return make_uint2(ua, ub);
  }
  // keep the first n (0..4) tokens of a V load, zero the rest
  static __device__ __forceinline__ void keep(VLoad& v, int n) {
    const uint64_t bits = n >= 4 ? ~0ull : ((1ull << (16 * n)) - 1ull);
    v.x &= static_cast<uint32_t>(bits);
    v.y &= static_cast<uint32_t>(bits >> 32);
  }
  // Two steps in one 32-deep product: lane (r, q) holds V tokens 4q .. 4q+3 of
  // step a then of step b (column 16 cb + r; v = {a, b}) and the same 8
  // tokens' weights of row r -- the contraction index k = 8q + e runs over
  // both steps.
  static __device__ __forceinline__ f32x4 pv2(const uint4& v, const uint4& p, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v),
                                                   __builtin_bit_cast(bf16x8, p), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint4 pack8(const float (&p)[8], float& sum) {
    const float a[4] = {p[0], p[1], p[2], p[3]};
    const float b[4] = {p[4], p[5], p[6], p[7]};
    const POp pa = pack(a, sum);
    const POp pb = pack(b, sum);
    return make_uint4(pa.x, pa.y, pb.x, pb.y);
  }
};

struct MmaF16 {
  static constexpr int kKBytes = 2;
  static constexpr int kKBits = 16;
  using KLoad = uint4;
  static constexpr int kVBytes = 2;
  static constexpr int kQOps = 1;
  using VLoad = uint2;
  using POp = uint2;
  static __device__ __forceinline__ f32x4 qk(const uint4& k, const uint4* q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q[0]), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(const VLoad& v, const POp& p, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, v),
                                                 __builtin_bit_cast(f16x4, p), c, 0, 0, 0);
  }
  static __device__ __forceinline__ POp pack(const float (&p)[4], float& sum) {
    const f16x2 a = {static_cast<_Float16>(p[0]), static_cast<_Float16>(p[1])};
    const f16x2 b = {static_cast<_Float16>(p[2]), static_cast<_Float16>(p[3])};
    sum += (static_cast<float>(a[0]) + static_cast<float>(a[1])) +
           (static_cast<float>(b[0]) + static_cast<float>(b[1]));
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
  }
  static __device__ __forceinline__ void keep(VLoad& v, int n) { MmaBF16::keep(v, n); }
  static __device__ __forceinline__ f32x4 pv2(const uint4& v, const uint4& p, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, v),
                                                  __builtin_bit_cast(f16x8, p), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint4 pack8(const float (&p)[8], float& sum) {
    const float a[4] = {p[0], p[1], p[2], p[3]};
    const float b[4] = {p[4], p[5], p[6], p[7]};
    const POp pa = pack(a, sum);
    const POp pb = pack(b, sum);
    return make_uint4(pa.x, pa.y, pb.x, pb.y);
  }
};

struct MmaF32 {
  static constexpr int kKBytes = 4;
  static constexpr int kKBits = 32;
  using KLoad = uint4;
  static constexpr int kVBytes = 4;
  static constexpr int kQOps = 1;
  using VLoad = uint4;  // 4 tokens of one V column
  struct POp {
    float p[4];
  };
  // a 16-byte chunk holds 4 elements: four 16x16x4 steps, element e of every
  // lane's chunk forming step e
  static __device__ __forceinline__ f32x4 qk(const uint4& k, const uint4* qp, f32x4 c) {
    const uint4 q = qp[0];
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.x), __uint_as_float(q.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.y), __uint_as_float(q.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.z), __uint_as_float(q.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.w), __uint_as_float(q.w), c, 0, 0, 0);
    return c;
  }
  // token 4q + e of the lane's V load meets weight e: step e pairs them
  static __device__ __forceinline__ f32x4 pv(const VLoad& v, const POp& p, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.x), p.p[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.y), p.p[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.z), p.p[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w), p.p[3], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ POp pack(const float (&p)[4], float& sum) {
    sum += (p[0] + p[1]) + (p[2] + p[3]);
    return POp{{p[0], p[1], p[2], p[3]}};
  }
  static __device__ __forceinline__ void keep(VLoad& v, int n) {
    if (n < 1) v.x = 0u;
    if (n < 2) v.y = 0u;
    if (n < 3) v.z = 0u;
    if (n < 4) v.w = 0u;
  }
};

// Int8 keys with float32 per-channel scales; values (and q, out) of the 16-bit
// type of VM.  A 16-byte K load brings 16 channels of one token: two 16x16x32
// f16 steps, the low 8 channels against q operand 0 and the high 8 against
// operand 1.  The B operand is q' = q * scale per channel (times a power of
// two per row, taken out again on the logits), rounded to f16; the codes
// convert to f16 exactly (biased by a constant the logit removes once per row,
// see codes()), so the matrix cores see exact values.
template <class VM>
struct MmaK8 {
  static constexpr int kKBytes = 1;
  static constexpr int kKBits = 8;
  using KLoad = uint4;
  static constexpr int kVBytes = 2;
  static constexpr int kQOps = 2;
  using VLoad = typename VM::VLoad;
  using POp = typename VM::POp;
  // 8 int8 codes (two words) -> f16x8, biased.  code ^ 0x80 is the
  // offset-binary byte u = code + 128, and the f16 with bits 0x5800 | u is
  // 128 + u / 8 = 144 + code / 8, exact (eight bits of a ten-bit mantissa).
  // The bias is not subtracted per code: the logit products sum
  // 144 Q + (1/8) sum_c q'_c code_c with Q = sum_c q'_c, so the kernel takes
  // the logit as 8 qs * sum - 1152 qs Q in one fused multiply-add (kCodeMul,
  // kCodeOffset; Q from the row's rounded operands).  The bias costs at most a
  // few units in the f32 sums' last places of 144 Q -- far below the f16
  // rounding of q' itself.
  static constexpr float kCodeMul = 8.f;
  static constexpr float kCodeOffset = 1152.f;
  static __device__ __forceinline__ f16x8 codes(uint32_t w0, uint32_t w1) {
    w0 ^= 0x80808080u;
    w1 ^= 0x80808080u;
    constexpr uint32_t kExp = 0x58585858u;
    const u32x4 h = {__builtin_amdgcn_perm(kExp, w0, 0x04010400u),
                     __builtin_amdgcn_perm(kExp, w0, 0x04030402u),
                     __builtin_amdgcn_perm(kExp, w1, 0x04010400u),
                     __builtin_amdgcn_perm(kExp, w1, 0x04030402u)};
    return __builtin_bit_cast(f16x8, h);
  }
  static __device__ __forceinline__ f32x4 qk(const uint4& k, const uint4* q, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes(k.x, k.y), __builtin_bit_cast(f16x8, q[0]), c,
                                               0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes(k.z, k.w), __builtin_bit_cast(f16x8, q[1]), c,
                                               0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4 pv(const VLoad& v, const POp& p, f32x4 c) {
    return VM::pv(v, p, c);
  }
  static __device__ __forceinline__ POp pack(const float (&p)[4], float& sum) {
    return VM::pack(p, sum);
  }
  static __device__ __forceinline__ void keep(VLoad& v, int n) { VM::keep(v, n); }
};

// 2-bit keys with float32 per-channel steps and zero points; values (and q,
// out) of the 16-bit type of VM.  One load per tile: lane (r, q) reads the
// D / 64 words of token r and channel group q (8 bytes at d 128, 4 at d 64),
// which hold channels 32 j + 8 q + e (e = 0..7) for all D / 32 logit steps j:
// step j is word j / 2, half j % 2 (bits 8 and up of the word, shifted down
// by 8, for half 1), and (word & (0x30003 << 2i)) keeps the codes of the pair
// e = 2i, 2i + 1 in place, at bits 2i and 16 + 2i.  Or-ing in 0x6400 makes each
// half the f16 1024 + code * 4^i (at most 1216: exact) -- no shift per pair.
// The B operand is q' = q * step per channel (times a power of two per row, as
// for int8 keys) times 4^-i for the elements of pair i, so the products are
// q'_c code_c plus the bias (see codes()); the zero points add the same
// scale * sum_c q_c z_c to every logit of a row (kept in qb).
template <class VM, int D>
struct MmaK2 {
  static constexpr int kKBytes = 0;  // sub-byte keys
  static constexpr int kKBits = 2;
  static constexpr int kVBytes = 2;
  static constexpr int kQOps = D / 32;  // B operands per K load (one load per tile)
  using KLoad = typename std::conditional<D == 128, uint2, uint32_t>::type;
  using VLoad = typename VM::VLoad;
  using POp = typename VM::POp;
  static __device__ __forceinline__ uint32_t word(const KLoad& k, int i) {
    if constexpr (D == 128) {
      return i == 0 ? k.x : k.y;
    } else {
      return k;
    }
  }
  // The 1024 bias of each half stays in: the products sum
  // 1024 Q + sum_c q'_c code_c (Q = sum_c of the rounded operands), and the
  // kernel subtracts 1024 qs Q once per row inside the fused multiply-add of
  // the logit (kCodeOffset).
  static constexpr float kCodeMul = 1.f;
  static constexpr float kCodeOffset = 1024.f;
  static __device__ __forceinline__ f16x8 codes(uint32_t w, int h) {
    const uint32_t x = h ? (w >> 8) : w;
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (x & (0x00030003u << (2 * i))) | 0x64006400u;
    return __builtin_bit_cast(f16x8, v);
  }
  static __device__ __forceinline__ f32x4 qk(const KLoad& k, const uint4* q, f32x4 c) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes(word(k, j / 2), j % 2),
                                                 __builtin_bit_cast(f16x8, q[j]), c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4 pv(const VLoad& v, const POp& p, f32x4 c) {
    return VM::pv(v, p, c);
  }
  static __device__ __forceinline__ POp pack(const float (&p)[4], float& sum) {
    return VM::pack(p, sum);
  }
  static __device__ __forceinline__ void keep(VLoad& v, int n) { VM::keep(v, n); }
};

// maximum / sum over the four lanes r, r+16, r+32, r+48 (lane-swap butterflies)
__device__ __forceinline__ float max_over_q(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_q(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Maxima of logits.  The logits that reach a row maximum are finite or -inf,
// never NaN (a slot past a row's limit is set to -inf first, whatever its key
// held), so the plain v_max instructions give the exact maximum.  fmaxf would
// also quiet a signalling NaN in every operand the compiler cannot trace to an
// arithmetic result -- after the masking branch and after each lane swap, one
// more instruction per operand (int8-key 8-token verify: 213.5 -> 196.5 us per
// launch, the other kernels unchanged).
__device__ __forceinline__ float lmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float lmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// the row's maximum over its four lanes r, r+16, r+32, r+48
__device__ __forceinline__ float lmax_over_q(float v) {
  const uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = lmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return lmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// physical blocks of one 16-token step (b == a for 16-token blocks)
struct Phys {
  int a, b;
};

// Wavefronts per SIMD the register allocation must leave room for (512
// registers per lane and SIMD): the ring of kDepth steps, the accumulators and
// the query operands of a lane fit 168 registers at d 128 with one chunk (three
// waves), 256 with two; float32 tiles are twice as large.
template <class M, int D, int kChunks, bool kLds>
constexpr int min_waves_per_simd() {
  if constexpr (M::kKBytes == 4) return D == 128 ? 2 : (kChunks == 1 ? 3 : 2);
  // the LDS ring reads two tiles per pass into registers
  if constexpr (kLds) return D == 128 ? 3 : 4;
  return D == 128 ? (kChunks == 1 ? 3 : 2) : (kChunks == 1 ? 5 : 3);
}

template <class M, class Tr, int D, int kWaves, int kChunks, bool kShared, int kBS,
          bool kWavePart, bool kLds = false, bool kPrefix = false>
__global__ __launch_bounds__(kWaves * 64, (min_waves_per_simd<M, D, kChunks, kLds>())) void decode_kernel(
    DecodeArgs a) {
  // kLds: four waves hold the four 16-row chunks of 64 rows and share each
  // step's tile through an LDS ring (see below); otherwise every wave holds all
  // kChunks chunks of the workgroup's rows and the waves split the steps.
  static_assert(!kLds || (kWaves == 4 && kChunks == 1 && !kWavePart), "LDS ring: 4 x 16 rows");
  static_assert(!kPrefix || !kLds, "shared prefix: register path");
  constexpr int kRowWaves = kLds ? 4 : 1;            // waves that split the rows
  constexpr int kStepWaves = kWaves / kRowWaves;     // waves that split the steps
  constexpr int kWgRows = 16 * kChunks * kRowWaves;  // rows of one workgroup
  // Sibling workgroups (kShared) read each tile through the XCD's L2 one after
  // another, so their loads must not carry the streaming hint.
  constexpr bool kStreamK = !kShared && (PA_DECODE_NT == 1 || PA_DECODE_NT == 2);
  constexpr bool kStreamV = !kShared && (PA_DECODE_NT == 1 || PA_DECODE_NT == 3);
  // K loads per tile: 1 KiB each (16-byte chunks / 4), or one smaller load
  // covering a 2-bit tile
  constexpr int kKLoads = D * M::kKBits / 512 > 0 ? D * M::kKBits / 512 : 1;
  constexpr int kQOps = kKLoads * M::kQOps;      // B operands of the logits per row
  constexpr int kColBlocks = D / 16;           // P.V output blocks of 16 columns
  constexpr int kPad = 4;                      // LDS row padding (floats)
  // kWavePart (split mode): each wave owns one whole partition and writes its
  // partial itself, so a workgroup covers kWaves consecutive partitions with
  // no merge through LDS; otherwise the waves share one partition's blocks.
  constexpr int kStride = kWavePart ? 1 : kStepWaves;  // logical-step stride of a wave
  using VLoad = typename M::VLoad;
  using KLoad = typename M::KLoad;

  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int qg = lane >> 4;
  const int wave = wave_id();
  const int rw = wave % kRowWaves;  // this wave's chunk of the workgroup's rows
  const int sw = wave / kRowWaves;  // this wave's share of the steps
  // kPrefix: the first a.shared_units workgroups take the prefix role -- the
  // partitions [0, a.shared_parts) of the prefix every table starts with,
  // for the rows of all sequences at once (as if the batch were one sequence
  // with a num_seqs-token query, read through table row 0, without a causal
  // limit); the others compute each sequence's partitions from a.part_offset.
  const bool prefix_role = kPrefix && static_cast<int>(blockIdx.x) < a.shared_units;
  const int T = prefix_role ? a.num_seqs : a.num_query_tokens;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int rows = T * group;  // (query token, query head) rows that read KV head g
  const int wgs = (rows + kWgRows - 1) / kWgRows;
  const int grid_parts = prefix_role ? a.shared_parts : a.num_parts;
  const int part_units = kWavePart ? (grid_parts + kWaves - 1) / kWaves : grid_parts;
  const int first_unit = kPrefix && !prefix_role ? a.shared_units : 0;
  const int role_units = kPrefix ? (prefix_role ? a.shared_units : gridDim.x - a.shared_units)
                                 : gridDim.x;
  const Unit u = unit_of(blockIdx.x - first_unit, role_units, wgs, part_units, a.num_kv_heads);
  const int gpart = kWavePart ? u.part * kWaves + wave : u.part;  // partition within the grid
  const int part = gpart + (prefix_role ? 0 : a.part_offset);
  const int g = u.kv_head;
  const int row0 = u.sibling * kWgRows + rw * (16 * kChunks);
  const int s = u.seq;
  if (kWavePart && gpart >= grid_parts) return;  // a wave past the last partition (no barriers)

  const int L = prefix_role ? a.shared_tokens : pa_clamp_len(a.context_lens[s], a.max_context_len);
  // causal reference: query token i sees the tokens [0, Lc - T + 1 + i); the
  // prefix role's rows see all L tokens
  const int Lc = prefix_role ? L + T - 1 : L;
  const int t_lo = part * a.partition_tokens;
  const int t_hi = min(L, t_lo + a.partition_tokens);
  // 16-token steps of the partition (a step is one 16-token block or two
  // 8-token blocks)
  const int blk_lo = t_lo / kStep;
  const int blk_hi = t_hi > t_lo ? (t_hi + kStep - 1) / kStep : blk_lo;
  // Query token i sees the tokens [0, Lc - T + 1 + i) (the draft is causal; one
  // query token sees the whole context).  Blocks that end past the smallest
  // limit of this wave's rows are masked row by row.
  const int t_hi_min = min(t_hi, Lc - T + 1 + row0 / group);

  // Per chunk c, lane l holds row row0 + 16 c + r: the B operands of its logits
  // (for 16-bit keys chunk 4j + qg of that row's query vector; zero for padding
  // rows), its token limit, the scale of its logits and its online-softmax state.
  uint4 qop[kChunks][kQOps];
  int row_hi[kChunks];
  float qs[kChunks];  // logits in log2 units: scale * log2(e) (and the quantised-key row factor)
  float qb[kChunks];  // 2-bit keys: the zero points' logit offset of the row (log2 units)
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int rho = row0 + 16 * c + r;
    const bool live = rho < rows;
    const int rr = live ? rho : rows - 1;  // padding rows read a live row, then drop it
    const int i = rr / group;
    const int hq = g * group + rr % group;
    const char* qrow = static_cast<const char*>(a.q) +
                       ((static_cast<size_t>(s) * T + i) * a.num_q_heads + hq) * D * M::kVBytes;
    qs[c] = a.scale * kLog2e;
    qb[c] = 0.f;
    if constexpr (M::kKBits >= 16) {
#pragma unroll
      for (int j = 0; j < kKLoads; ++j) {
        const uint4 v = reinterpret_cast<const uint4*>(qrow)[4 * j + qg];
        qop[c][j] = live ? v : make_uint4(0u, 0u, 0u, 0u);
      }
    } else if constexpr (M::kKBits == 8) {
      // int8 keys: load j brings channels 16 (4j + qg) .. + 15 of a token; the
      // matching q' = q * k_scale, scaled by 2^e so that the row's largest
      // |q'| lies in [2^13, 2^14) (full f16 precision whatever the scales),
      // and 2^-e folded into the logit scale.
      const float* ks = a.k_scale + static_cast<size_t>(g) * D;
      float qp[kKLoads][16];
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < kKLoads; ++j) {
        const int ch = 16 * (4 * j + qg);
        float e[16];
        Tr::unpack(reinterpret_cast<const uint4*>(qrow)[ch / 8], e);
        Tr::unpack(reinterpret_cast<const uint4*>(qrow)[ch / 8 + 1], e + 8);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float4 sc4 = reinterpret_cast<const float4*>(ks + ch)[t];
          qp[j][4 * t + 0] = e[4 * t + 0] * sc4.x;
          qp[j][4 * t + 1] = e[4 * t + 1] * sc4.y;
          qp[j][4 * t + 2] = e[4 * t + 2] * sc4.z;
          qp[j][4 * t + 3] = e[4 * t + 3] * sc4.w;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) mx = fmaxf(mx, fabsf(qp[j][t]));
      }
      mx = max_over_q(mx);  // the row's four lanes
      int ex = 0;
      if (mx > 0.f) {
        (void)frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
      }
      const float up = ldexpf(1.f, 14 - ex);
      qs[c] *= ldexpf(1.f, ex - 14);
      float qsum = 0.f;
#pragma unroll
      for (int j = 0; j < kKLoads; ++j) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          f16x8 h;
#pragma unroll
          for (int t = 0; t < 8; ++t) h[t] = static_cast<_Float16>(qp[j][8 * hh + t] * up);
#pragma unroll
          for (int t = 0; t < 8; ++t) qsum += static_cast<float>(h[t]);
          const uint4 v = __builtin_bit_cast(uint4, h);
          qop[c][2 * j + hh] = live ? v : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      qsum = sum_over_q(live ? qsum : 0.f);
      qb[c] = -M::kCodeOffset * qs[c] * qsum;
      qs[c] *= M::kCodeMul;
    } else {
      // 2-bit keys: operand j holds channels 32 j + 8 qg .. + 7 of q' = q * step,
      // scaled as for int8 keys; the lane's share of sum_c q_c z_c joins the
      // other three lanes of the row.
      const float* ks = a.k_scale + static_cast<size_t>(g) * D;
      const float* kz = a.k_zero + static_cast<size_t>(g) * D;
      float qp[kQOps][8];
      float mx = 0.f, zb = 0.f;
#pragma unroll
      for (int j = 0; j < kQOps; ++j) {
        const int ch = 32 * j + 8 * qg;
        float e[8];
        Tr::unpack(reinterpret_cast<const uint4*>(qrow)[ch / 8], e);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float4 sc4 = reinterpret_cast<const float4*>(ks + ch)[t];
          const float4 z4 = reinterpret_cast<const float4*>(kz + ch)[t];
          qp[j][4 * t + 0] = e[4 * t + 0] * sc4.x;
          qp[j][4 * t + 1] = e[4 * t + 1] * sc4.y;
          qp[j][4 * t + 2] = e[4 * t + 2] * sc4.z;
          qp[j][4 * t + 3] = e[4 * t + 3] * sc4.w;
          zb += (e[4 * t + 0] * z4.x + e[4 * t + 1] * z4.y) + (e[4 * t + 2] * z4.z + e[4 * t + 3] * z4.w);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) mx = fmaxf(mx, fabsf(qp[j][t]));
      }
      mx = max_over_q(mx);  // the row's four lanes
      zb = sum_over_q(zb);
      int ex = 0;
      if (mx > 0.f) {
        (void)frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
      }
      const float up = ldexpf(1.f, 14 - ex);
      qb[c] = zb * qs[c];
      qs[c] *= ldexpf(1.f, ex - 14);
      float qsum = 0.f;
#pragma unroll
      for (int j = 0; j < kQOps; ++j) {
        f16x8 h;
#pragma unroll
        for (int t = 0; t < 8; ++t) h[t] = static_cast<_Float16>(qp[j][t] * up * ldexpf(1.f, -2 * (t >> 1)));
#pragma unroll
        for (int t = 0; t < 8; ++t) qsum += static_cast<float>(h[t]);
        const uint4 v = __builtin_bit_cast(uint4, h);
        qop[c][j] = live ? v : make_uint4(0u, 0u, 0u, 0u);
      }
      qsum = sum_over_q(live ? qsum : 0.f);
      qb[c] -= M::kCodeOffset * qs[c] * qsum;
      qs[c] *= M::kCodeMul;
    }
    row_hi[c] = live ? min(t_hi, Lc - T + 1 + i) : t_hi;
  }

  float m[kChunks];     // running maximum (log2 units) of row r, shared by its 4 lanes
  float lsum[kChunks];  // this lane's share of the running sum
  f32x4 acc[kChunks][kColBlocks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    m[c] = -INFINITY;
    lsum[c] = 0.f;
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) acc[c][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* __restrict__ trow = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
  const char* __restrict__ kbase = static_cast<const char*>(a.k_pool);
  const char* __restrict__ vbase = static_cast<const char*>(a.v_pool);

  // Physical blocks of 16-token step jb, read through the scalar cache: one
  // 16-token block, or two 8-token blocks (the second one repeats the first
  // when the context ends inside the first: its tokens are masked anyway).
  const int live_blocks = (L + kBS - 1) / kBS;
  auto physical = [&](int jb) {
    // every caller's step index is wave-uniform: the ids come through the
    // scalar cache, and waiting for them leaves the tile loads in flight
    Phys p;
    if constexpr (kBS == 16) {
      p.a = p.b = pa_physical_block_uniform(trow, jb, a.num_blocks);
    } else {
      p.a = pa_physical_block_uniform(trow, 2 * jb, a.num_blocks);
      p.b = 2 * jb + 1 < live_blocks ? pa_physical_block_uniform(trow, 2 * jb + 1, a.num_blocks)
                                     : p.a;
    }
    return p;
  };

  // Per-lane tile pointers of a step and the addresses of its K operand j and
  // V operand cb.  8-token tiles: K token r of the step is token r % 8 of
  // block r / 8 (the lane's chunk 4j + qg at [chunk][r % 8]: 512 contiguous
  // bytes per half wave); V tokens 4qg .. 4qg+3 are tokens 4 (qg % 2) .. of
  // block qg / 2.
  struct TilePtrs {
    const KLoad* kt;
    const VLoad* vt;
  };
  auto tile_ptrs = [&](Phys ph) {
    TilePtrs p;
    if constexpr (kBS == 16) {
      const size_t tile = pa_tile_offset(ph.a, g, a.num_kv_heads, D, 16);  // elements
      p.kt = reinterpret_cast<const KLoad*>(kbase + tile * M::kKBits / 8);
      p.vt = reinterpret_cast<const VLoad*>(vbase + tile * M::kVBytes);
    } else {
      const size_t ta = pa_tile_offset(ph.a, g, a.num_kv_heads, D, 8);
      const size_t tb = pa_tile_offset(ph.b, g, a.num_kv_heads, D, 8);
      p.kt = reinterpret_cast<const KLoad*>(kbase + (r < 8 ? ta : tb) * M::kKBits / 8);
      p.vt = reinterpret_cast<const VLoad*>(vbase + (qg < 2 ? ta : tb) * M::kVBytes);
    }
    return p;
  };
  auto k_at = [&](const TilePtrs& p, int j) {
    return kBS == 16 ? p.kt + 64 * j + lane : p.kt + (4 * j + qg) * 8 + (r & 7);
  };
  auto v_at = [&](const TilePtrs& p, int cb) {
    return kBS == 16 ? p.vt + (16 * cb + r) * 4 + qg : p.vt + (16 * cb + r) * 2 + (qg & 1);
  };
  auto load = [&](Phys ph, KLoad (&kr)[kKLoads], VLoad (&vr)[kColBlocks]) {
    const TilePtrs p = tile_ptrs(ph);
#pragma unroll
    for (int j = 0; j < kKLoads; ++j) kr[j] = load16<kStreamK>(k_at(p, j));
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) vr[cb] = load16<kStreamV>(v_at(p, cb));
  };

  auto consume = [&](int jb, const KLoad (&kr)[kKLoads], VLoad (&vr)[kColBlocks]) {
    const int tok0 = jb * kStep + 4 * qg;  // first token of this lane's four
    if ((jb + 1) * kStep > t_hi) {          // V rows past the partition (wave-uniform test)
      const int n = min(max(t_hi - tok0, 0), 4);
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) M::keep(vr[cb], n);
    }
    const bool masked = (jb + 1) * kStep > t_hi_min;  // wave-uniform
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kKLoads; ++j) sc = M::qk(kr[j], &qop[c][j * M::kQOps], sc);
      float x[4];
      if constexpr (M::kKBits < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = fmaf(sc[i], qs[c], qb[c]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = sc[i] * qs[c];
      }
      if (masked) {
        const int n = min(max(row_hi[c] - tok0, 0), 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i >= n) x[i] = -INFINITY;
      }
      const float bmax = lmax_over_q(lmax3(x[0], x[1], lmax(x[2], x[3])));
      const bool raise = bmax > m[c] + kSlack;
      if (__builtin_amdgcn_ballot_w64(raise)) {  // wave-uniform
        const float alpha = raise ? __builtin_amdgcn_exp2f(m[c] - bmax) : 1.f;  // 0 on a first block
        m[c] = raise ? bmax : m[c];
        lsum[c] *= alpha;
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) acc[c][cb] *= alpha;
      }
      const float mref = m[c] == -INFINITY ? 0.f : m[c];  // a row that has seen no token yet
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mref);
      const typename M::POp pop = M::pack(p, lsum[c]);
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) acc[c][cb] = M::pv(vr[cb], pop, acc[c][cb]);
    }
  };

  // The wave's steps are jb(i) = first + i * kStride, i in [0, n) (kStride =
  // kWaves when the waves share a partition, 1 when the wave owns it).  A ring
  // of kDepth register sets: step i is consumed while steps i+1 .. i+kDepth-1
  // are in flight; the physical id of the step to load next is read one step
  // before its tile loads are issued.  Every load below is issued
  // unconditionally on its path (the last steps get one branch per count), so
  // the wait before each consume covers exactly the step consumed: a load that
  // may or may not have been issued would make the compiler wait for every
  // load in flight, the next steps' included.
  KLoad kr[kDepth][kKLoads];
  VLoad vr[kDepth][kColBlocks];
  const int first = blk_lo + (kWavePart ? 0 : sw);
  const int n = first < blk_hi ? (blk_hi - first + kStride - 1) / kStride : 0;
  auto step_of = [&](int i) { return first + i * kStride; };
  if constexpr (kLds) {
    // The four waves hold the four 16-row chunks of the workgroup's 64 rows
    // and walk the same steps, two at a time.  Each step's tile is read from
    // memory once: wave w loads K operands w, w + 4, ... and V operands w,
    // w + 4, ... (for every lane) of both steps of a pair, writes them to a
    // two-pair LDS ring, and after one barrier every wave reads both tiles back
    // as its own operands.
    constexpr int kKS = (kKLoads + 3) / 4;
    constexpr int kVS = (kColBlocks + 3) / 4;
    // K: [pair slot * 2 + step][operand][lane]; V: [pair slot][operand][lane]
    // holding the lane's operand of step a in its low and of step b in its high
    // 8 bytes, so one 16-byte read returns the 32-deep P.V operand, and one
    // 16-byte store per lane writes both steps' shares.
    __shared__ uint4 lds_k[4][kKLoads][64];
    __shared__ uint4 lds_v[2][kColBlocks][64];
    uint4 sk[2][kKS];
    VLoad sv[2][kVS];
    auto stage_k = [&](const TilePtrs& p, uint4 (&k)[kKS]) {
#pragma unroll
      for (int i = 0; i < kKS; ++i) k[i] = load16<kStreamK>(k_at(p, min(wave + 4 * i, kKLoads - 1)));
    };
    auto stage_v = [&](const TilePtrs& p, VLoad (&v)[kVS]) {
#pragma unroll
      for (int i = 0; i < kVS; ++i)
        v[i] = load16<kStreamV>(v_at(p, min(wave + 4 * i, kColBlocks - 1)));
    };
    // Steps ja and ja + 1 in one pass: their logits, one raise decision and one
    // set of rounded weights for the 32 tokens, and P.V as one 16x16x32 product
    // per 16 columns (pv2).  A step past the partition is entirely masked.
    auto consume_pair = [&](int ja, const uint4 (&ka)[kKLoads], const uint4 (&kb)[kKLoads],
                            uint4 (&vv)[kColBlocks]) {
      const int tok_a = ja * kStep + 4 * qg;  // first token of this lane's four in step ja
      const int tok_b = tok_a + kStep;
      if ((ja + 2) * kStep > t_hi) {  // V rows past the partition (wave-uniform test)
        const int na = min(max(t_hi - tok_a, 0), 4);
        const int nb = min(max(t_hi - tok_b, 0), 4);
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) {
          VLoad va = make_uint2(vv[cb].x, vv[cb].y);
          VLoad vb = make_uint2(vv[cb].z, vv[cb].w);
          M::keep(va, na);
          M::keep(vb, nb);
          vv[cb] = make_uint4(va.x, va.y, vb.x, vb.y);
        }
      }
      f32x4 sa = {0.f, 0.f, 0.f, 0.f};
      f32x4 sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kKLoads; ++j) {
        sa = M::qk(ka[j], &qop[0][j * M::kQOps], sa);
        sb = M::qk(kb[j], &qop[0][j * M::kQOps], sb);
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = sa[i] * qs[0];
        x[4 + i] = sb[i] * qs[0];
      }
      if ((ja + 2) * kStep > t_hi_min) {  // wave-uniform
        const int na = min(max(row_hi[0] - tok_a, 0), 4);
        const int nb = min(max(row_hi[0] - tok_b, 0), 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= na) x[i] = -INFINITY;
          if (i >= nb) x[4 + i] = -INFINITY;
        }
      }
      const float bmax =
          lmax_over_q(lmax3(lmax3(x[0], x[1], x[2]), lmax3(x[3], x[4], x[5]), lmax(x[6], x[7])));
      const bool raise = bmax > m[0] + kSlack;
      if (__builtin_amdgcn_ballot_w64(raise)) {  // wave-uniform
        const float alpha = raise ? __builtin_amdgcn_exp2f(m[0] - bmax) : 1.f;  // 0 on a first step
        m[0] = raise ? bmax : m[0];
        lsum[0] *= alpha;
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) acc[0][cb] *= alpha;
      }
      const float mref = m[0] == -INFINITY ? 0.f : m[0];  // a row that has seen no token yet
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mref);
      const uint4 pop = M::pack8(p, lsum[0]);
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) acc[0][cb] = M::pv2(vv[cb], pop, acc[0][cb]);
    };
    const int nl = blk_hi - blk_lo;  // workgroup-uniform: every wave walks every step
    if (nl > 0) {
      // the first pair, in the order every pass issues its loads (the waits
      // below count on it): K of step a, K of step b, V of both
      {
        const TilePtrs pa = tile_ptrs(physical(blk_lo));
        const TilePtrs pb = tile_ptrs(physical(blk_lo + min(1, nl - 1)));
        stage_k(pa, sk[0]);
        stage_k(pb, sk[1]);
        stage_v(pa, sv[0]);
        stage_v(pb, sv[1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      Phys next_a = physical(blk_lo + min(2, nl - 1));
      Phys next_b = physical(blk_lo + min(3, nl - 1));
      // pair i (steps 2i, 2i + 1) in ring slot `slot`: publish its staged tile
      // shares, stage pair i + 1 (the last step again past the end: no branch,
      // so the waits before the ring writes stay exact), barrier, read both
      // tiles back, compute.  The loads of a pair are issued in the order K of
      // step a, K of step b, V of both: each K share is written and re-staged
      // before the next wait, and the two steps' V shares go out as one 16-byte
      // store per operand, so at every wait the next loads are already in
      // flight and no LDS store is narrower than 16 bytes (8-byte stores at a
      // 16-byte stride conflict on the banks).  With fewer than four operands of
      // a kind, two waves load and write the same one: equal values, so the
      // duplicate write is harmless.
      auto lds_pair = [&](int i, int slot) {
        const TilePtrs pa = tile_ptrs(next_a);
        const TilePtrs pb = tile_ptrs(next_b);
#pragma unroll
        for (int t = 0; t < kKS; ++t) lds_k[2 * slot][min(wave + 4 * t, kKLoads - 1)][lane] = sk[0][t];
        stage_k(pa, sk[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kKS; ++t) lds_k[2 * slot + 1][min(wave + 4 * t, kKLoads - 1)][lane] = sk[1][t];
        stage_k(pb, sk[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kVS; ++t)
          lds_v[slot][min(wave + 4 * t, kColBlocks - 1)][lane] =
              make_uint4(sv[0][t].x, sv[0][t].y, sv[1][t].x, sv[1][t].y);
        stage_v(pa, sv[0]);
        stage_v(pb, sv[1]);
        __builtin_amdgcn_sched_barrier(0);
        next_a = physical(blk_lo + min(2 * i + 4, nl - 1));
        next_b = physical(blk_lo + min(2 * i + 5, nl - 1));
        __syncthreads();
        uint4 ka[kKLoads], kb[kKLoads], vv[kColBlocks];
#pragma unroll
        for (int j = 0; j < kKLoads; ++j) {
          ka[j] = lds_k[2 * slot][j][lane];
          kb[j] = lds_k[2 * slot + 1][j][lane];
        }
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb) vv[cb] = lds_v[slot][cb][lane];
        if (row0 < rows) consume_pair(blk_lo + 2 * i, ka, kb, vv);
      };
      const int np = (nl + 1) / 2;  // workgroup-uniform
      int i = 0;
      for (; i + 2 <= np; i += 2) {
        lds_pair(i, 0);
        lds_pair(i + 1, 1);
      }
      if (i < np) lds_pair(i, 0);  // pairs alternate slots: an even index takes slot 0
    }
    // every lane of a row holds the row's whole sum: one share, for the
    // four-lane sum below
  }
  if (!kLds && n > 0) {  // wave-uniform
    // prologue: steps 0 .. kDepth-2 (an index past the last step reloads it)
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) load(physical(step_of(min(d, n - 1))), kr[d], vr[d]);
    Phys next_phys = physical(step_of(min(kDepth - 1, n - 1)));
    int base = 0;
    // steady state: every step entering the ring exists
    for (; base + 2 * kDepth - 1 <= n; base += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int in = base + u + kDepth - 1;  // the step entering the ring
        load(next_phys, kr[(u + kDepth - 1) % kDepth], vr[(u + kDepth - 1) % kDepth]);
        next_phys = physical(step_of(min(in + 1, n - 1)));
        consume(step_of(base + u), kr[u], vr[u]);
      }
    }
    // the last r = n - base <= 2 kDepth - 2 steps (base is a multiple of
    // kDepth, so step base + u sits in ring slot u % kDepth), one branch per r
    // so that every load inside it is unconditional as well
    const int r = n - base;
#pragma unroll
    for (int R = 1; R <= 2 * kDepth - 2; ++R) {
      if (r == R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const int in = u + kDepth - 1;
          if (in < R) {
            load(next_phys, kr[in % kDepth], vr[in % kDepth]);
            if (in + 1 < R) next_phys = physical(step_of(base + in + 1));
          }
          consume(step_of(base + u), kr[u % kDepth], vr[u % kDepth]);
        }
      }
    }
  }

  // Here partials are stored with the streaming hint: they are read once, by
  // the merge kernel, and plain stores that stay in L2 cost this launch more
  // than their bytes, all waves storing at once at the end (70B batch at
  // 512-token partitions: decode 182.3 -> 172-176 us; 163 us with no stores at
  // all; 32K batch 88.4 -> 86-87.6 us).  Rows stored whole through LDS, or
  // written through to memory (agent- or system-scope stores), measured no
  // better or worse; the merged stores of the LDS path below stay plain (the
  // hint cost the shared-prefix batch 69 -> 73 us there).
  if constexpr (kWavePart || kLds) {
    // every row of this wave lives in this wave alone (its own partition, or
    // its own chunk of the workgroup's rows): normalise in registers and write
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int rho = row0 + 16 * c + r;
      const float ls = sum_over_q(lsum[c]);  // all lanes take part
      const bool seen = m[c] != -INFINITY;
      const float inv = seen ? 1.f / ls : 0.f;
      const size_t row = (static_cast<size_t>(s) * T + rho / group) * a.num_q_heads +
                         g * group + rho % group;
      if (a.write_partials) {
        if (qg == 0 && rho < rows)
          a.lse_part[row * a.part_stride + part] = seen ? (m[c] + __log2f(ls)) * kLn2 : -INFINITY;
        if (rho < rows) {
          float* op = a.o_part + (row * a.part_stride + part) * D + 4 * qg;
#pragma unroll
          for (int cb = 0; cb < kColBlocks; ++cb)
            __builtin_nontemporal_store(acc[c][cb] * inv, reinterpret_cast<f32x4*>(op + 16 * cb));
        }
      } else if (rho < rows) {
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) Tr::store(a.out, row * D + 16 * cb + 4 * qg + i, acc[c][cb][i] * inv);
      }
    }
    return;
  }

  // merge the waves through LDS, one chunk of 16 rows at a time, and write
  __shared__ float sm_o[kWaves][16][D + kPad];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int nh = min(16, rows - (row0 + 16 * c));  // live rows of this chunk
    if (nh <= 0) break;                              // workgroup-uniform
    const float ls = sum_over_q(lsum[c]);
    if (c > 0) __syncthreads();  // the previous chunk's merge has read LDS
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb)
      *reinterpret_cast<f32x4*>(&sm_o[wave][r][16 * cb + 4 * qg]) = acc[c][cb];
    if (qg == 0) {
      sm_m[wave][r] = m[c];
      sm_l[wave][r] = ls;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nh * D; idx += kWaves * 64) {
      const int h = idx / D;
      const int col = idx % D;
      float M_ = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M_ = fmaxf(M_, sm_m[w][h]);
      float o = 0.f, lse = -INFINITY;
      if (M_ != -INFINITY) {
        float lsw = 0.f, os = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = __builtin_amdgcn_exp2f(sm_m[w][h] - M_);  // 0 for an idle wave
          lsw = fmaf(sm_l[w][h], f, lsw);
          os = fmaf(sm_o[w][h][col], f, os);
        }
        o = os / lsw;
        lse = (M_ + __log2f(lsw)) * kLn2;
      }
      const int rho = row0 + 16 * c + h;
      const size_t row = (static_cast<size_t>(s) * T + rho / group) * a.num_q_heads +
                         g * group + rho % group;
      if (a.write_partials) {
        a.o_part[(row * a.part_stride + part) * D + col] = o;
        if (col == 0) a.lse_part[row * a.part_stride + part] = lse;
      } else {
        Tr::store(a.out, row * D + col, o);
      }
    }
  }
}

// Partitions of at least this many tokens get 8 wavefronts per workgroup (each
// wave still streams a long run of blocks, and a ragged batch finishes more
// evenly); shorter ones get 4.  2-bit keys always get 4: a step carries 4.5 KiB
// instead of 8, and three 4-wave workgroups per compute unit keep more of them
// in flight than one of 8 (measured on the 70B batch: 97.1 -> 92.9 us; ring
// depths 3 and 4 changed nothing).  Waves holding two row chunks (17 to 32 rows
// per KV head) get 4 as well: the same waves fit a compute unit as two 4-wave
// workgroups as one of 8, and the smaller ones start and finish independently
// and merge four waves' results instead of eight (70B batch verifying a
// 4-token draft: 178 -> 171 us; with int8 keys 148 -> 137 us).
constexpr int kWideTokens = 4096;

// One wave per partition needs at least this many partitions per sequence and
// this many workgroups.
constexpr int kWavePartMin = 8;
constexpr unsigned kWavePartUnits = 256;

// Row chunks per workgroup (at most PA_MAX_CHUNKS; two measured best on
// MI355X: four chunks hold too much state per lane to keep enough waves
// resident): the rows of one KV head in as few workgroups as allowed; when they
// need more, the workgroups become siblings on one XCD.
#ifndef PA_MAX_CHUNKS
#define PA_MAX_CHUNKS 2
#endif
int chunks_for(int rows) {
  const int c = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  return c < PA_MAX_CHUNKS ? c : PA_MAX_CHUNKS;
}

template <class M, class Tr, int D, int kChunks, bool kShared, int kBS>
hipError_t launch_cs(const DecodeArgs& a, int wgs, hipStream_t stream) {
  const unsigned units = a.num_kv_heads * wgs * a.num_seqs;
  // Split mode over many partitions: one wave per partition, four partitions
  // per workgroup, when that still gives every wave a partition and the chip
  // enough workgroups (measured on the 32K batch: 512-token partitions 93.1 ->
  // 85.7 us; with two partitions per sequence half the waves would idle).
  const unsigned groups = (a.num_parts + 3) / 4;
  if (a.write_partials && a.num_parts >= kWavePartMin && units * groups >= kWavePartUnits) {
    hipLaunchKernelGGL((decode_kernel<M, Tr, D, 4, kChunks, kShared, kBS, true>),
                       dim3(units * groups), dim3(4 * 64), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid(units * a.num_parts);
  // Only one-chunk waves take 8-wave workgroups (two chunks: see kWideTokens;
  // four hold 64 rows of state per lane, which only 4 waves fit unspilled).
  if constexpr (kChunks == 1) {
    if (M::kKBits != 2 && a.partition_tokens >= kWideTokens) {
      hipLaunchKernelGGL((decode_kernel<M, Tr, D, 8, kChunks, kShared, kBS, false>), grid,
                         dim3(8 * 64), 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_kernel<M, Tr, D, 4, kChunks, kShared, kBS, false>), grid,
                     dim3(4 * 64), 0, stream, a);
  return hipGetLastError();
}

template <class M, class Tr, int D, int kChunks>
hipError_t launch_c(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.num_query_tokens * (a.num_q_heads / a.num_kv_heads);
  const int wgs = (rows + 16 * kChunks - 1) / (16 * kChunks);
  if (a.block_size == 8) {
    if (wgs > 1) return launch_cs<M, Tr, D, kChunks, true, 8>(a, wgs, stream);
    return launch_cs<M, Tr, D, kChunks, false, 8>(a, wgs, stream);
  }
  if (wgs > 1) return launch_cs<M, Tr, D, kChunks, true, 16>(a, wgs, stream);
  return launch_cs<M, Tr, D, kChunks, false, 16>(a, wgs, stream);
}

// More than 32 rows per KV head with 16-bit keys: workgroups of 64 rows whose
// four waves share each tile through LDS (measured on the 70B batch against
// two-chunk siblings: 6-, 8- and 16-token drafts 234 -> 202, 242 -> 215 and
// 402 -> 366 us).  Up to 32 rows one two-chunk workgroup per KV head stays:
// with two of the four waves idle the LDS workgroup is no faster there and
// varies from launch to launch.  Int8 keys keep the register path: in this
// scheme every wave converts the whole key tile for its one chunk, which
// measured slower.
template <class M, class Tr, int D, bool kShared, int kBS>
hipError_t launch_lds_s(const DecodeArgs& a, int wgs, hipStream_t stream) {
  const dim3 grid(a.num_kv_heads * wgs * a.num_seqs * a.num_parts);
  hipLaunchKernelGGL((decode_kernel<M, Tr, D, 4, 1, kShared, kBS, false, true>), grid,
                     dim3(4 * 64), 0, stream, a);
  return hipGetLastError();
}
template <class M, class Tr, int D>
hipError_t launch_lds(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.num_query_tokens * (a.num_q_heads / a.num_kv_heads);
  const int wgs = (rows + 63) / 64;
  if (a.block_size == 8)
    return wgs > 1 ? launch_lds_s<M, Tr, D, true, 8>(a, wgs, stream)
                   : launch_lds_s<M, Tr, D, false, 8>(a, wgs, stream);
  return wgs > 1 ? launch_lds_s<M, Tr, D, true, 16>(a, wgs, stream)
                 : launch_lds_s<M, Tr, D, false, 16>(a, wgs, stream);
}

template <class M, class Tr, int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (M::kKBytes == 2) {
    if (a.num_query_tokens * (a.num_q_heads / a.num_kv_heads) > 32)
      return launch_lds<M, Tr, D>(a, stream);
  }
  if constexpr (M::kKBytes == 4 && D == 128) {
    // an 8 KiB float32 tile fills the registers already: one chunk per workgroup
    return launch_c<M, Tr, D, 1>(a, stream);
  } else {
    switch (chunks_for(a.num_query_tokens * (a.num_q_heads / a.num_kv_heads))) {
      case 1: return launch_c<M, Tr, D, 1>(a, stream);
#if PA_MAX_CHUNKS >= 4
      case 4: return launch_c<M, Tr, D, 4>(a, stream);
#endif
      default: return launch_c<M, Tr, D, 2>(a, stream);
    }
  }
}

template <class M, class Tr>
hipError_t launch_dim(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_t<M, Tr, 64>(a, stream) : launch_t<M, Tr, 128>(a, stream);
}
template <class VM, class Tr>
hipError_t launch_dim_k2(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_t<MmaK2<VM, 64>, Tr, 64>(a, stream)
                          : launch_t<MmaK2<VM, 128>, Tr, 128>(a, stream);
}

// Shared-prefix split launch: one grid, prefix-role workgroups first (the
// prefix partitions of every KV head, for all sequences' rows: siblings of
// 16 * kChunks rows placed on one XCD, so each prefix tile leaves HBM once and
// the siblings read it from that XCD's L2), then one workgroup per (sequence,
// KV head, private partition), spread over all XCDs.  Both roles run the same
// register-path kernel (the prefix role's rows are only wider in number).
// Measured on the shared-prefix batch (128 sequences, 1024 shared + U[16,
// 1024] private tokens, 32/8 heads; decode kernel, us): loads without the
// streaming hint, so that siblings find the prefix in L2: 61.9 -> 57.2 at
// 1024-token partitions, 69.9 -> 62.1 at 512; one wave per partition up to
// 512 tokens (private units are short): 62.1 -> 57.2 at 512, 73.2 -> 62.2 at
// 256.  pa_decode on the same batch: 70.4 (1024-token partitions).
constexpr int kPrefixWavePartTokens = 512;
template <class M, class Tr, int D, int kChunks, int kBS>
hipError_t launch_prefix_c(DecodeArgs a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int64_t prefix_wgs = (static_cast<int64_t>(a.num_seqs) * group + 16 * kChunks - 1) / (16 * kChunks);
  const int64_t private_wgs = (group + 16 * kChunks - 1) / (16 * kChunks);
  constexpr bool kPlain = true;  // kShared: loads without the streaming hint
  if (a.partition_tokens <= kPrefixWavePartTokens) {
    // one wave per partition, four partitions per workgroup, in both roles
    const int64_t shared = a.num_kv_heads * prefix_wgs * ((a.shared_parts + 3) / 4);
    const int64_t total = shared + static_cast<int64_t>(a.num_kv_heads) * private_wgs * a.num_seqs *
                                       ((a.num_parts + 3) / 4);
    a.shared_units = static_cast<int32_t>(shared);
    hipLaunchKernelGGL((decode_kernel<M, Tr, D, 4, kChunks, kPlain, kBS, true, false, true>),
                       dim3(static_cast<uint32_t>(total)), dim3(4 * 64), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t shared = a.num_kv_heads * prefix_wgs * a.shared_parts;
  const int64_t total = shared + static_cast<int64_t>(a.num_kv_heads) * private_wgs * a.num_seqs * a.num_parts;
  a.shared_units = static_cast<int32_t>(shared);
  if (a.partition_tokens >= kWideTokens) {
    hipLaunchKernelGGL((decode_kernel<M, Tr, D, 8, kChunks, kPlain, kBS, false, false, true>),
                       dim3(static_cast<uint32_t>(total)), dim3(8 * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<M, Tr, D, 4, kChunks, kPlain, kBS, false, false, true>),
                       dim3(static_cast<uint32_t>(total)), dim3(4 * 64), 0, stream, a);
  }
  return hipGetLastError();
}
template <class M, class Tr, int D>
hipError_t launch_prefix_t(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  // Two row chunks per workgroup as soon as the prefix role has more than 32
  // rows (every sequence's rows of a KV head): half the sibling workgroups,
  // each prefix tile read half as often from the XCD's L2 (shared-prefix batch,
  // 128 sequences x 4 rows, 1024-token partitions: 59.2 -> 56.5 us per step;
  // at 512-token partitions, one wave per partition, one chunk stays ahead:
  // 60.3 vs 63.5).  Float32 tiles at d 128 fill the registers with one chunk.
  const bool two = (group > 16 || (static_cast<int64_t>(a.num_seqs) * group > 32 &&
                                   a.partition_tokens > kPrefixWavePartTokens)) &&
                   !(M::kKBytes == 4 && D == 128);
  if (a.block_size == 8)
    return two ? launch_prefix_c<M, Tr, D, 2, 8>(a, stream) : launch_prefix_c<M, Tr, D, 1, 8>(a, stream);
  return two ? launch_prefix_c<M, Tr, D, 2, 16>(a, stream) : launch_prefix_c<M, Tr, D, 1, 16>(a, stream);
}
template <class M, class Tr>
hipError_t launch_prefix_dim(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_prefix_t<M, Tr, 64>(a, stream)
                          : launch_prefix_t<M, Tr, 128>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case PA_F32: return launch_dim<MmaF32, F32>(a, stream);
    case PA_F16: return launch_dim<MmaF16, F16>(a, stream);
    case PA_K8_F16: return launch_dim<MmaK8<MmaF16>, F16>(a, stream);
    case PA_K8_BF16: return launch_dim<MmaK8<MmaBF16>, BF16>(a, stream);
    case PA_K2_F16: return launch_dim_k2<MmaF16, F16>(a, stream);
    case PA_K2_BF16: return launch_dim_k2<MmaBF16, BF16>(a, stream);
    default: return launch_dim<MmaBF16, BF16>(a, stream);
  }
}

hipError_t launch_decode_shared_prefix(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case PA_F32: return launch_prefix_dim<MmaF32, F32>(a, stream);
    case PA_F16: return launch_prefix_dim<MmaF16, F16>(a, stream);
    case PA_K8_F16: return launch_prefix_dim<MmaK8<MmaF16>, F16>(a, stream);
    case PA_K8_BF16: return launch_prefix_dim<MmaK8<MmaBF16>, BF16>(a, stream);
    case PA_K2_F16:
      return a.head_dim == 64 ? launch_prefix_t<MmaK2<MmaF16, 64>, F16, 64>(a, stream)
                              : launch_prefix_t<MmaK2<MmaF16, 128>, F16, 128>(a, stream);
    case PA_K2_BF16:
      return a.head_dim == 64 ? launch_prefix_t<MmaK2<MmaBF16, 64>, BF16, 64>(a, stream)
                              : launch_prefix_t<MmaK2<MmaBF16, 128>, BF16, 128>(a, stream);
    default: return launch_prefix_dim<MmaBF16, BF16>(a, stream);
  }
}

}  // namespace pa
