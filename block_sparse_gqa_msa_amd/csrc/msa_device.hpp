// msa_device.hpp -- device-side building blocks shared by the MSA kernels (gfx950 only).
//
// Matrix-core conventions used throughout (CDNA 16x16 MFMA tiles, wave64):
//   A operand  (16 x K):  lane l holds row (l % 16), K-elements of lane group g = l / 16
//   B operand  (K x 16):  lane l holds column (l % 16), the same K-elements of group g
//   C/D (16 x 16 fp32):   lane l holds rows 4*g + i (i = 0..3) of column (l % 16)
// A "fragment" is the 8 K-elements one lane feeds for a 32-wide K chunk: K-elements
// 8*g + 0..7 of the chunk. For bf16 that is one v_mfma_f32_16x16x32_bf16; for fp32 it
// is eight v_mfma_f32_16x16x4_f32, the j-th of which takes element j of every lane.
// Because A and B always use the same K-element -> (lane group, slot) assignment, any
// fixed permutation of the K axis inside a chunk gives the same product; the attention
// kernel relies on this to feed P^T straight from the accumulator layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage tag for bf16 tensors (raw 16-bit patterns in memory).
struct bf16_t {
  uint16_t bits;
};

template <typename E> struct Frag;
template <> struct Frag<bf16_t> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

// Load the 8 consecutive elements at p (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ bf16x8 load_frag(const bf16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ f32x8 load_frag(const float *p) {
  const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
  f32x4 a = q[0], b = q[1];
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x8 zero_frag(const bf16_t *) { return bf16x8{}; }
__device__ __forceinline__ f32x8 zero_frag(const float *) { return f32x8{}; }

// acc += A(16 x 32-chunk) * B(32-chunk x 16)
__device__ __forceinline__ f32x4 mfma_chunk(bf16x8 a, bf16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_chunk(f32x8 a, f32x8 b, f32x4 acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Value of lane (l ^ 32) and (l ^ 16) via the gfx950 half-wave / row swaps: each
// returns the pair {own, partner} in some order, so max/sum of the pair reduces.
__device__ __forceinline__ float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Maximum of scores for the index branch's pooling: the IEEE 754-2019 maximum (gfx950's
// v_maximum3_f32). For values that are not NaN it is the same maximum as fmaxf, -0 below
// +0; unlike fmaxf it needs no quieting pass (a v_max_f32 x, x, x per operand that the
// compiler cannot prove canonical, such as matrix-core results and lane swaps), which
// had been a third of the pooling's instructions.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Transposing max-reduction over the four lane groups: given per-lane values v0..v3 (one
// per 16-column N-tile), returns in lane group g the maximum of v_g over all four groups.
// Uses v_permlane32_swap (x <-> upper half of the other operand) then v_permlane16_swap.
__device__ __forceinline__ float max_groups_transpose(float v0, float v1, float v2, float v3) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  const float t0 = smax(__uint_as_float(a[0]), __uint_as_float(a[1]));  // N-tile 0 (lo) / 2 (hi)
  const float t1 = smax(__uint_as_float(b[0]), __uint_as_float(b[1]));  // N-tile 1 (lo) / 3 (hi)
  auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(t0), __float_as_uint(t1), false, false);
  return smax(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Max of N values as a chain of three-input maxima (v_maximum3_f32).
template <int N>
__device__ __forceinline__ float max_chain(const float (&v)[N]) {
  static_assert(N >= 2, "max_chain needs two values");
  float m = smax(v[0], v[1]);
#pragma unroll
  for (int i = 2; i + 1 < N; i += 2) m = smax(smax(m, v[i]), v[i + 1]);
  if constexpr (N % 2 == 1) m = smax(m, v[N - 1]);
  return m;
}

// Reduce over the four lane groups (l % 16 fixed).
__device__ __forceinline__ float max_groups(float v) { return max_xor32(max_xor16(v)); }
__device__ __forceinline__ float sum_groups(float v) { return sum_xor32(sum_xor16(v)); }

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Order-preserving map of a float that is not NaN (infinities included) to uint32:
// a > b <=> key(a) > key(b) and a == b <=> key(a) == key(b); -0 is first made +0 (the sum
// below), the same score, so that equal scores tie. Key 0 is below every such float and
// marks "no candidate".
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Pin a loaded value: an empty asm that reads and writes it. A load whose result only
// some lanes use can otherwise be moved under a branch on those lanes, and loads under
// branches are issued one at a time (each waits for the one before). Issue every load of
// a batch first, then pin them all.
template <typename T>
__device__ __forceinline__ void pin(T &x) {
  asm volatile("" : "+v"(x));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }
// Number of set bits of m below this lane.
__device__ __forceinline__ int rank_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m));
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m));
  return v;
}

// Dynamic chunk assignment for the persistent KV-outer kernels: the first gridDim.x chunks
// go by block index, every later one to the workgroup that claims it. A workgroup claims
// its next chunk when it starts one, so the atomic's round trip overlaps the chunk. Every
// processed chunk makes exactly one claim, so the claim that returns n_chunks - 1 is the
// kernel's last: it resets the counter (zeroed by the plan) for the next launch. Static
// striding left whole rounds of workgroups idle behind the slowest: chunk costs vary with
// list lengths.
__device__ __forceinline__ int claim_next(int32_t *claim, int n_chunks) {
  const int c = atomicAdd(claim, 1);
  if (c == n_chunks - 1) atomicExch(claim, 0);
  return c + (int)gridDim.x;
}

}  // namespace msa
