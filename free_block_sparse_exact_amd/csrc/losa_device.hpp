// Device-side helpers shared by the gfx950 kernels: vector types, the bf16
// matrix-core tile product, loads, wave reductions and the XCD-aware
// workgroup mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace losa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// 16x16x32 bf16 matrix-core product: D = A (16 x 32) * B (32 x 16) + C.
// Lane l feeds row (l & 15) of A and column (l & 15) of B with eight
// k-elements each; the k-elements must be laid out identically in A and B
// (any such layout gives the same contraction).  D: lane l holds column
// (l & 15), rows 4 * (l >> 4) + [0, 4).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;  // round to nearest even (v_cvt_pk_bf16_f32)
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }

// Eight fp32 values -> bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                        float a7) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  return __builtin_convertvector((f32x8{a0, a1, a2, a3, a4, a5, a6, a7}), bf16x8);
}

// Sum of eight bf16 probabilities exactly as they enter a P.V product, so a
// softmax normaliser matches its numerator (v_dot2 against (1, 1)).
__device__ __forceinline__ float sum_bf16x8(bf16x8 p) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float s = __builtin_amdgcn_fdot2_f32_bf16(p.s01, ones, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(p.s23, ones, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(p.s45, ones, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(p.s67, ones, s, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the four 16-lane rows of a wave (lane = 16 * row + column)
// on gfx950's lane swaps, vector instructions that need no LDS permute:
// v_permlane32_swap(a, b) returns (a.lo, b.lo) and (a.hi, b.hi) by 32-lane
// halves, v_permlane16_swap(a, b) returns (a.r0, b.r0, a.r2, b.r2) and
// (a.r1, b.r1, a.r3, b.r3) by 16-lane rows.  Every lane must be active.
// The sums add the same pairs in the same grouping as the xor-16-then-32
// (or 32-then-16) exchange they replace, so results are bit-identical.
__device__ __forceinline__ float swap_sum32(float a, float b) {  // lower lanes: a + a', upper: b' + b
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {  // even rows: a + a', odd rows: b' + b
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane (row g, column c) gets v[g] summed over the four rows at column c:
// each lane ends with the total of "its own" value of the four.
__device__ __forceinline__ float rows_sum_own(const float (&v)[4]) {
  return swap_sum16(swap_sum32(v[0], v[2]), swap_sum32(v[1], v[3]));
}

// x summed (maximised) over the four rows: every lane gets its column's total.
__device__ __forceinline__ float rows_sum(float x) {
  const float y = swap_sum16(x, x);
  return swap_sum32(y, y);
}

__device__ __forceinline__ float rows_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, kWave);
    v = v > w ? v : w;
  }
  return v;
}

// Workgroup ids are handed to the 8 XCDs round-robin; map them so that each
// XCD works through one contiguous range of tasks (neighbouring tasks share
// K/V rows, so they then share that XCD's L2).  A bijection on [0, n).
__device__ __forceinline__ int xcd_task(int bid, int n) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd;
  const int local = bid / kXcd;
  const int base = n / kXcd;
  const int rem = n % kXcd;
  const int start = xcd * base + (xcd < rem ? xcd : rem);
  return start + local;
}

// Workgroup id -> task for work lists whose neighbouring tasks read the same
// data (rows of one head, in the budget order): consecutive blocks of 32
// tasks are dealt to the 8 XCDs round-robin, so at any time each XCD's CUs
// run 32 neighbouring tasks (sharing that XCD's L2) while every XCD still
// draws from the whole list (keeping uneven budgets balanced across XCDs).
// A bijection on [0, n); the tail beyond the last whole group of 8*32 tasks
// keeps the identity.
__device__ __forceinline__ int xcd_block_task(int bid, int n) {
  constexpr int kXcd = 8, kBlock = 32, kGroup = kXcd * kBlock;
  const int full = n / kGroup * kGroup;
  if (bid >= full) return bid;
  const int xcd = bid % kXcd, local = bid / kXcd;
  return (local / kBlock) * kGroup + xcd * kBlock + (local % kBlock);
}

}  // namespace losa
