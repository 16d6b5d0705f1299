// Device helpers shared by the indexer kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kHeadDim = 128;
constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// float32 pair -> OCP e4m3fn codes: round to nearest even, saturate to +-448, keep the
// sign (-0 and negative underflow give 0x80).  The format (bias 7, 3 mantissa bits,
// subnormals m * 2^-9, largest finite 448 = 2^8 * 1.75) rounds the fp32 mantissa to
// 3 bits in the normal range and |x| * 2^9 to an integer below 2^-6; |x| >= 464 (the
// tie between 448 and the non-finite next step) saturates.  gfx950's packed
// conversion to OCP fp8 rounds the same way in range, so the value is clamped to
// +-448 (which saturates exactly as above) and converted in hardware; the clamped
// conversion was compared with that definition, written out in integer arithmetic,
// on every fp32 pattern of magnitude <= 500 and both signs, without a mismatch.
// Returns the codes of (a, b) in bits 0..7 and 8..15 (one conversion per pair).
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f), cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
// max over groups of `W` consecutive lanes (W a power of two <= 64)
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows that hold the
// same column of a 16x16 MFMA accumulator), with the gfx950 row-swap permutes:
// permlane16_swap(x, x) yields the pair (x of rows 0,0,2,2 ; x of rows 1,1,3,3), and
// permlane32_swap the pair (halves 0,0 ; halves 1,1).  Pure VALU, no LDS round trip.
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reduce-scatter over the four 16-lane rows for four 16-key groups at once.  p_g
// holds, in lane l, a partial sum for key l%16 of group g over the heads of lane-row
// l/16; the result in lane l is the full sum (all four rows) for key l%16 of group
// l/16, i.e. key l of the 64-key span.  permlane32_swap(a, b) leaves
// (a.lo, b.lo | a.hi, b.hi) so a.lo + a.hi pairs rows (0,2) and (1,3): the low half
// keeps groups 0 and 1, the high half groups 2 and 3; one permlane16_swap then pairs
// the remaining rows.  3 swaps and 3 adds for 64 keys.
__device__ __forceinline__ float rows4_reduce_scatter(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float s13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// max(x, 0) on the bit pattern: non-negative floats order like signed integers and
// every negative float (including -0) is a negative integer, so one v_max_i32 gives
// the ReLU with +0 for every non-positive input.  (fmaxf would first canonicalise
// its operand in IEEE mode, a second instruction.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// Workgroup barrier that orders LDS only: wait for this wave's LDS operations, then
// s_barrier.  __syncthreads() adds a workgroup-scope release fence, which on gfx9
// drains every outstanding vector-memory load as well, so global prefetches could
// never stay in flight across it.  The memory clobber keeps the compiler from moving
// memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// number of set bits of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace dsa
