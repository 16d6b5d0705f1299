// Index-K store and the contiguous fp8 quantiser.
//
// Store chain per token ("The Pivot: A Single Edit That Finally Fixed DeepSeek V4's
// Long-Context Recall Failure", "The Reasoning Behind the Edit": the unfused key
// path normalises, applies RoPE and rotates, and writes the cache last; ROCm/ATOM
// issue 1507, "Root cause found" and "Where": interleaved RoPE on the trailing
// rope_dim, then the Walsh-Hadamard rotation the key must share with the query),
// fused into one pass over registers:
//   RMSNorm -> RoPE -> 128-point Hadamard -> fp8 absmax quantise (or bf16 round)
//   -> scatter into the paged cache.
// The query preparation runs the same chain on every query vector (the query must
// carry the key's rotation, issue 1507 "Root cause found"; its RoPE + Hadamard +
// fp8 preparation, "Where") and writes dense bf16 and/or fp8 outputs.
//
// The store runs one wavefront per token; lane l owns elements 2l and 2l+1, which is exactly one
// interleaved RoPE pair, and the Hadamard butterflies run on index bit 0 inside the
// lane and on bits 1..6 across lanes (lane bit b-1), so the whole chain stays in two
// registers per lane.  The token is tiny (256 B in, 132 B out): the kernel is
// launch- and latency-bound, never bandwidth-bound, at the sizes of a decode or
// chunked-prefill step.  The quantisers of dense vectors (query preparation, the
// contiguous quantiser) map a vector onto 16 lanes instead, below.
#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr uint32_t kNorm = 1u, kRope = 2u, kHadamard = 4u;

// RoPE coefficients of this lane's pair (elements 2*lane, 2*lane+1) at `position`:
// pair i = lane - (128 - rope_dim)/2 of the trailing rope_dim rotates by
// theta = position * rope_base^(-2i/rope_dim); lanes below the rotated range get
// (1, 0).  ln_step = -(2/rope_dim) ln(rope_base) comes from the host, so the
// frequency is one double exp.  The angle is formed in double (positions reach ~1M,
// where a float angle is ~0.06 rad off), reduced modulo 2 pi by Cody and Waite's
// method with 2 pi split into a double and its remainder (each product folded in
// with one fma), and the remainder, |r| <= pi, goes to single-precision sin/cos.
__device__ __forceinline__ void rope_coeffs(int lane, double ln_step, int rope_dim, int32_t position,
                                            float& c, float& s) {
  c = 1.0f;
  s = 0.0f;
  const int o = kHeadDim - rope_dim;
  if (2 * lane >= o) {
    const int i = lane - o / 2;
    const double theta = (double)position * exp((double)i * ln_step);
    const double kTwoPiHi = 6.283185307179586232;       // 2 pi rounded to double
    const double kTwoPiLo = 2.4492935982947064e-16;     // 2 pi - kTwoPiHi
    const double kInvTwoPi = 0.15915494309189535;
    const double k = rint(theta * kInvTwoPi);
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, theta));
    sincosf((float)r, &s, &c);
  }
}

// The per-vector chain on this lane's pair (y0, y1) = elements (2*lane, 2*lane+1),
// with the pair's RoPE coefficients (c, s) (used with kRope).
__device__ __forceinline__ void vector_chain(float& y0, float& y1, int lane, uint32_t flags, float eps,
                                             float c, float s) {
  if (flags & kNorm) {
    const float ss = wave_sum(y0 * y0 + y1 * y1);
    const float r = 1.0f / sqrtf(ss / 128.0f + eps);
    y0 *= r;
    y1 *= r;
  }
  if (flags & kRope) {
    const float a = y0, b = y1;
    y0 = a * c - b * s;
    y1 = a * s + b * c;
  }
  if (flags & kHadamard) {
    // Sylvester-order H_128 = H_2 (x) ... (x) H_2: one butterfly per index bit.
    const float a = y0 + y1, b = y0 - y1;
    y0 = a;
    y1 = b;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float p0 = __shfl_xor(y0, m), p1 = __shfl_xor(y1, m);
      const bool upper = (lane & m) != 0;
      y0 = upper ? (p0 - y0) : (y0 + p0);
      y1 = upper ? (p1 - y1) : (y1 + p1);
    }
    const float inv_sqrt128 = 0.0883883476483184405501f;
    y0 *= inv_sqrt128;
    y1 *= inv_sqrt128;
  }
}

// fp8 absmax quantisation of the vector held as (y0, y1) pairs across the wave:
// amax = max|y|, s = amax/448 (correctly rounded; 1 when amax < 2^-100), codes e4m3(y/s).
__device__ __forceinline__ uint32_t quantise_pair(float y0, float y1, float& s) {
  const float amax = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
  s = amax / 448.0f;  // correctly rounded division (no fast-math)
  if (amax < 0x1p-100f) s = 1.0f;
  return e4m3_encode2(y0 / s, y1 / s);
}

// DPP lane selects within 16-lane rows (quad_perm [1,0,3,2], [2,3,0,1], [3,2,1,0],
// the 8-lane half mirror, and rotations of the row by 4 and 8 lanes).
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kQuadRev = 0x1B, kHalfMirror = 0x141;
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xF, 0xF, true));
}
// Value held by lane l ^ M of the same 16-lane row, M = 1, 2, 4, 8: xor 4 is xor 3
// inside the quad followed by the half mirror (xor 7); xor 8 is the rotation by 8.
template <int M>
__device__ __forceinline__ float row_xor(float v) {
  if constexpr (M == 1) return dpp<kQuadXor1>(v);
  else if constexpr (M == 2) return dpp<kQuadXor2>(v);
  else if constexpr (M == 4) return dpp<kHalfMirror>(dpp<kQuadRev>(v));
  else {
    static_assert(M == 8, "row_xor: M must be 1, 2, 4 or 8");
    return dpp<kRowRor8>(v);
  }
}
// Sum and max over a 16-lane row, left in every lane: the quad by two xors, then the
// row's four quads by rotations of 4 and 8 lanes.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowRor4>(v);
  return v + dpp<kRowRor8>(v);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowRor4>(v));
  return fmaxf(v, dpp<kRowRor8>(v));
}

// A value with the e4m3 code of RN32(y / s), given r = RN32(1 / s).  The product
// y * r carries two roundings of relative size 2^-24 against the quotient's one, so it
// lies within 3 units in the last place of RN32(y / s), and both take the same e4m3
// code unless an e4m3 rounding step lies that close.  The steps of the normal range
// are the fp32 values whose low 20 mantissa bits are 0x80000 (the tie of the 3-bit
// mantissa round, 464 included); those below 2^-6 are the subnormal ties.  A product
// within 4 units of a normal-range step, or below 2^-6, is redone with the correctly
// rounded division.
__device__ __forceinline__ float quotient_for_e4m3(float y, float s, float r) {
  const float q = y * r;
  const uint32_t a = __float_as_uint(q) & 0x7FFFFFFFu;
  if (a < 0x3C800000u || (a & 0xFFFFFu) - 0x7FFFCu <= 8u) return y / s;
  return q;
}

// fp8 absmax quantisation of a vector held as 8 consecutive elements per lane over
// a 16-lane row: the scale s = RN32(amax / 448) (1 when amax < 2^-100) and the codes
// e4m3(RN32(f_i / s)) packed little-endian into two words.
__device__ __forceinline__ void quantise8(const float (&f)[8], uint32_t& lo, uint32_t& hi, float& s) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = row16_max(m);
  s = m / 448.0f;  // correctly rounded division (no fast-math)
  if (m < 0x1p-100f) s = 1.0f;
  const float r = 1.0f / s;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = quotient_for_e4m3(f[i], s, r);
  lo = e4m3_encode2(q[0], q[1]) | (e4m3_encode2(q[2], q[3]) << 16);
  hi = e4m3_encode2(q[4], q[5]) | (e4m3_encode2(q[6], q[7]) << 16);
}

// e2m1 code of v (bit 3 = sign): the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to
// the even mantissa bit, saturating at 6.  Counting the thresholds passed, strict at
// the ties that round down (0.25, 1.25, 2.5, 5) and inclusive at those that round up
// (0.75, 1.75, 3.5), gives the code directly.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// MXFP4 quantisation of the vector held as (y0, y1) pairs across the wave: the 16
// lanes of DPP row g hold the 32-element block g.  Shared exponent
// e = floor(log2(amax)) - 2 within [-127, 127] (0 for an all-zero block); codes of
// y * 2^-e (exact: a power-of-two scaling).  Returns this lane's code byte (element
// 2*lane in the low nibble) and the block's e8m0 byte e + 127.
__device__ __forceinline__ uint32_t quantise_mxfp4_pair(float y0, float y1, uint32_t& e8) {
  const float amax = row16_max(fmaxf(fabsf(y0), fabsf(y1)));
  int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 2 : 0;
  e = min(max(e, -127), 127);
  e8 = (uint32_t)(e + 127);
  return e2m1_code(ldexpf(y0, -e)) | (e2m1_code(ldexpf(y1, -e)) << 4);
}

// kKind: 0 bf16 cache, 1 fp8 (e4m3 + fp32 scale), 2 MXFP4 (e2m1 + e8m0 per 32)
template <int kKind>
__global__ __launch_bounds__(256) void index_k_store_kernel(
    const uint16_t* __restrict__ x, int64_t n, const int32_t* __restrict__ pos,
    const int64_t* __restrict__ slots, uint8_t* __restrict__ base, int bs, int64_t num_blocks,
    uint32_t flags, float eps, double ln_step, int rope_dim, float* __restrict__ dbg) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;  // uniform per wave

  const uint32_t pair = reinterpret_cast<const uint32_t*>(x + t * kHeadDim)[lane];
  float y0 = bf16_lo(pair), y1 = bf16_hi(pair);
  float c = 1.0f, s = 0.0f;
  if (flags & kRope) rope_coeffs(lane, ln_step, rope_dim, pos[t], c, s);
  vector_chain(y0, y1, lane, flags, eps, c, s);
  if (dbg) reinterpret_cast<float2*>(dbg + t * kHeadDim)[lane] = make_float2(y0, y1);

  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_blocks * bs) return;  // uniform per wave
  const int64_t blk = slot / bs, off = slot - blk * bs;
  if constexpr (kKind == 1) {
    float s;
    const uint32_t c = quantise_pair(y0, y1, s);
    uint8_t* blkp = base + blk * (int64_t)bs * 132;
    reinterpret_cast<uint16_t*>(blkp + off * kHeadDim)[lane] = (uint16_t)c;
    if (lane == 0) reinterpret_cast<float*>(blkp + (int64_t)bs * kHeadDim)[off] = s;
  } else if constexpr (kKind == 2) {
    // block layout: [bs][64] code bytes, then [bs][4] e8m0 bytes (68 B per token)
    uint32_t e8;
    const uint32_t c = quantise_mxfp4_pair(y0, y1, e8);
    uint8_t* blkp = base + blk * (int64_t)bs * 68;
    blkp[off * 64 + lane] = (uint8_t)c;
    if ((lane & 15) == 0) blkp[(int64_t)bs * 64 + off * 4 + (lane >> 4)] = (uint8_t)e8;
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(base + (blk * bs + off) * 256);
    dst[lane] = f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16);
  }
}

// Query preparation: the store chain on every (row, head) vector of q [rows][heads][128],
// all heads of row r at positions[r]; outputs bf16 rows and/or fp8 codes + scales.
// A query row is 64 vectors at the decode and prefill shapes, so the vector is mapped
// onto a 16-lane row instead of the whole wave: lane `sub` holds elements
// 8*sub .. 8*sub+7 (one 16-byte load), the four rows of a wave take four heads at once,
// and a wave prepares IT such groups of heads of ONE query row, all rotated by the
// same RoPE angles, which the wave forms once (lane l computes pair l, then each lane
// gathers the four pairs it holds).  Interleaved RoPE pairs and Hadamard index bits
// 0..2 stay inside a lane; bits 3..6 are lane bits 0..3 and go through DPP exchanges.
template <int IT>
__global__ __launch_bounds__(256) void q_prep_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int heads, int wpr, const int32_t* __restrict__ pos,
    uint32_t flags, float eps, double ln_step, int rope_dim, uint16_t* __restrict__ out_bf16,
    uint8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ dbg) {
  const int lane = lane_id();
  const int sub = lane & 15;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t row = wid / wpr;
  if (row >= rows) return;  // uniform per wave
  const int h0 = (int)(wid - row * wpr) * (4 * IT) + (lane >> 4);

  uint4 raw[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int h = min(h0 + 4 * it, heads - 1);  // rows past the last head redo it, unstored
    raw[it] = reinterpret_cast<const uint4*>(x + (row * heads + h) * kHeadDim)[sub];
  }
  float rc[4] = {1.0f, 1.0f, 1.0f, 1.0f}, rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (flags & kRope) {
    float c, s;
    rope_coeffs(lane, ln_step, rope_dim, pos[row], c, s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rc[j] = __shfl(c, 4 * sub + j);
      rs[j] = __shfl(s, 4 * sub + j);
    }
  }

#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint4 u = raw[it];
    float f[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                  bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
    if (flags & kNorm) {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
      ss = row16_sum(ss);
      const float r = 1.0f / sqrtf(ss / 128.0f + eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] *= r;
    }
    if (flags & kRope) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = f[2 * j], b = f[2 * j + 1];
        f[2 * j] = a * rc[j] - b * rs[j];
        f[2 * j + 1] = a * rs[j] + b * rc[j];
      }
    }
    if (flags & kHadamard) {
      // Sylvester-order H_128: one butterfly (a, b) -> (a + b, a - b) per index bit
#pragma unroll
      for (int b = 1; b < 8; b <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i & b) continue;
          const float a0 = f[i], a1 = f[i | b];
          f[i] = a0 + a1;
          f[i | b] = a0 - a1;
        }
      }
      // bits 3..6 (lane bits 0..3): the butterfly gives the lower lane own + partner
      // and the upper partner - own; each lane forms own + c * partner instead (c = -1
      // on the upper lane, one fma with the exchanged operand), which is the negation
      // of the upper result.  The lanes paired at one bit carry equal signs from the
      // earlier bits, so after the four levels a lane holds (-1)^popcount(lane bits)
      // times its outputs, undone in the final scaling.
      const float c1 = (sub & 1) ? -1.0f : 1.0f, c2 = (sub & 2) ? -1.0f : 1.0f;
      const float c4 = (sub & 4) ? -1.0f : 1.0f, c8 = (sub & 8) ? -1.0f : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fmaf(row_xor<1>(f[i]), c1, f[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fmaf(row_xor<2>(f[i]), c2, f[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fmaf(row_xor<4>(f[i]), c4, f[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fmaf(row_xor<8>(f[i]), c8, f[i]);
      const float scale = (__builtin_popcount(sub) & 1) ? -0.0883883476483184405501f : 0.0883883476483184405501f;
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] *= scale;
    }
    uint32_t lo = 0, hi = 0;
    float sc = 1.0f;
    if (codes) quantise8(f, lo, hi, sc);  // group-wide: every row runs it, stored or not

    const int h = h0 + 4 * it;
    if (h < heads) {
      const int64_t v = row * heads + h;
      if (dbg) {
        float4* d = reinterpret_cast<float4*>(dbg + v * kHeadDim) + 2 * sub;
        d[0] = make_float4(f[0], f[1], f[2], f[3]);
        d[1] = make_float4(f[4], f[5], f[6], f[7]);
      }
      if (out_bf16) {
        uint4 o;
        o.x = f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16);
        o.y = f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16);
        o.z = f32_to_bf16_rne(f[4]) | (f32_to_bf16_rne(f[5]) << 16);
        o.w = f32_to_bf16_rne(f[6]) | (f32_to_bf16_rne(f[7]) << 16);
        reinterpret_cast<uint4*>(out_bf16 + v * kHeadDim)[sub] = o;
      }
      if (codes) {
        reinterpret_cast<uint2*>(codes + v * kHeadDim)[sub] = make_uint2(lo, hi);
        if (sub == 0) scales[v] = sc;
      }
    }
  }
}

// Contiguous per-vector quantiser: 16 lanes per vector, 8 elements (one 16-byte
// load) per lane, 4 vectors per wave, 16 vectors per 256-thread workgroup.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x,
                                                        int64_t n_vec, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int64_t v = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool live = v < n_vec;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (live) raw = reinterpret_cast<const uint4*>(x + v * kHeadDim)[sub];
  const float f[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                      bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  uint32_t lo, hi;
  float s;
  quantise8(f, lo, hi, s);
  if (live) {
    reinterpret_cast<uint2*>(codes + v * kHeadDim)[sub] = make_uint2(lo, hi);
    if (sub == 0) scales[v] = s;
  }
}

// -(2/rope_dim) ln(rope_base): the log-frequency step between RoPE pairs (0 when
// RoPE is off and the parameters are unchecked).
double rope_step(float rope_base, int rope_dim) {
  if (!(rope_base > 0.0f) || rope_dim <= 0) return 0.0;
  return -2.0 / (double)rope_dim * std::log((double)rope_base);
}

}  // namespace

hipError_t launch_store(const uint16_t* x, int64_t n, const int32_t* pos, const int64_t* slots,
                        const KCache& c, uint32_t flags, float eps, float rope_base, int rope_dim,
                        float* dbg, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const double ln_step = rope_step(rope_base, rope_dim);
  const dim3 grid((unsigned)((n + 3) / 4)), block(256);
  if (c.dtype == 2)
    hipLaunchKernelGGL(index_k_store_kernel<1>, grid, block, 0, s, x, n, pos, slots, c.base,
                       c.block_size, c.num_blocks, flags, eps, ln_step, rope_dim, dbg);
  else if (c.dtype == 3)
    hipLaunchKernelGGL(index_k_store_kernel<2>, grid, block, 0, s, x, n, pos, slots, c.base,
                       c.block_size, c.num_blocks, flags, eps, ln_step, rope_dim, dbg);
  else
    hipLaunchKernelGGL(index_k_store_kernel<0>, grid, block, 0, s, x, n, pos, slots, c.base,
                       c.block_size, c.num_blocks, flags, eps, ln_step, rope_dim, dbg);
  return hipGetLastError();
}

hipError_t launch_q_prep(const uint16_t* x, int64_t n_vec, int heads, const int32_t* pos, uint32_t flags,
                         float eps, float rope_base, int rope_dim, uint16_t* out_bf16, uint8_t* codes,
                         float* scales, float* dbg, hipStream_t s) {
  if (n_vec == 0) return hipSuccess;
  const int64_t rows = n_vec / heads;
  const double ln_step = rope_step(rope_base, rope_dim);
  // small calls: one group of four heads per wave (most waves in flight); large
  // ones: four groups per wave, so the RoPE angles are formed once per 16 heads
  const bool big = n_vec >= (1 << 16);
  const int per_wave = big ? 16 : 4;
  const int wpr = (int)(((int64_t)heads + per_wave - 1) / per_wave);
  const int64_t blocks = (rows * wpr + 3) / 4;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  if (big)
    hipLaunchKernelGGL(q_prep_kernel<4>, grid, block, 0, s, x, rows, heads, wpr, pos, flags, eps, ln_step,
                       rope_dim, out_bf16, codes, scales, dbg);
  else
    hipLaunchKernelGGL(q_prep_kernel<1>, grid, block, 0, s, x, rows, heads, wpr, pos, flags, eps, ln_step,
                       rope_dim, out_bf16, codes, scales, dbg);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n_vec, uint8_t* codes, float* scales,
                            hipStream_t s) {
  if (n_vec == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_vec + 15) / 16)), block(256);
  hipLaunchKernelGGL(quant_fp8_kernel, grid, block, 0, s, x, n_vec, codes, scales);
  return hipGetLastError();
}

}  // namespace dsa
