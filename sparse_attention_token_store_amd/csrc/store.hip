// Index-K store and the contiguous fp8 quantiser.
//
// Store chain per token ("The Pivot: A Single Edit That Finally Fixed DeepSeek V4's
// Long-Context Recall Failure", "The Reasoning Behind the Edit": normalise, RoPE and
// rotate before the store; ROCm/ATOM issue 1507, "Root cause found" and "Where":
// interleaved RoPE on the trailing rope_dim, then the Walsh-Hadamard rotation the
// key must share with the query), fused into one pass over registers:
//   RMSNorm -> RoPE -> 128-point Hadamard -> fp8 absmax quantise (or bf16 round)
//   -> scatter into the paged cache.
//
// One wavefront per token; lane l owns elements 2l and 2l+1, which is exactly one
// interleaved RoPE pair, and the Hadamard butterflies run on index bit 0 inside the
// lane and on bits 1..6 across lanes (lane bit b-1), so the whole chain stays in two
// registers per lane.  The token is tiny (256 B in, 132 B out): the kernel is
// launch- and latency-bound, never bandwidth-bound, at the sizes of a decode or
// chunked-prefill step.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr uint32_t kNorm = 1u, kRope = 2u, kHadamard = 4u;

template <bool kFp8>
__global__ __launch_bounds__(256) void index_k_store_kernel(
    const uint16_t* __restrict__ x, int64_t n, const int32_t* __restrict__ pos,
    const int64_t* __restrict__ slots, uint8_t* __restrict__ base, int bs, int64_t num_blocks,
    uint32_t flags, float eps, float rope_base, int rope_dim, float* __restrict__ dbg) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n) return;  // uniform per wave

  const uint32_t pair = reinterpret_cast<const uint32_t*>(x + t * kHeadDim)[lane];
  float y0 = bf16_lo(pair), y1 = bf16_hi(pair);

  if (flags & kNorm) {
    const float ss = wave_sum(y0 * y0 + y1 * y1);
    const float r = 1.0f / sqrtf(ss / 128.0f + eps);
    y0 *= r;
    y1 *= r;
  }
  if (flags & kRope) {
    const int o = kHeadDim - rope_dim;
    if (2 * lane >= o) {
      const int i = lane - o / 2;
      // angle in double: positions reach ~1M, where a float angle is ~0.06 rad off
      const double inv_freq = pow((double)rope_base, -2.0 * (double)i / (double)rope_dim);
      const double theta = (double)pos[t] * inv_freq;
      double sn, cs;
      sincos(theta, &sn, &cs);
      const float c = (float)cs, s = (float)sn;
      const float a = y0, b = y1;
      y0 = a * c - b * s;
      y1 = a * s + b * c;
    }
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
  if (dbg) reinterpret_cast<float2*>(dbg + t * kHeadDim)[lane] = make_float2(y0, y1);

  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_blocks * bs) return;  // uniform per wave
  const int64_t blk = slot / bs, off = slot - blk * bs;
  if constexpr (kFp8) {
    const float amax = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
    float s = amax / 448.0f;  // correctly rounded division (no fast-math)
    if (amax < 0x1p-100f) s = 1.0f;
    const uint32_t c0 = e4m3_encode(y0 / s), c1 = e4m3_encode(y1 / s);
    uint8_t* blkp = base + blk * (int64_t)bs * 132;
    reinterpret_cast<uint16_t*>(blkp + off * kHeadDim)[lane] = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) reinterpret_cast<float*>(blkp + (int64_t)bs * kHeadDim)[off] = s;
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(base + (blk * bs + off) * 256);
    dst[lane] = f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16);
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
  float f[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  const float amax = group_max<16>(m);
  float s = amax / 448.0f;
  if (amax < 0x1p-100f) s = 1.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= e4m3_encode(f[i] / s) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= e4m3_encode(f[4 + i] / s) << (8 * i);
  if (live) {
    reinterpret_cast<uint2*>(codes + v * kHeadDim)[sub] = make_uint2(lo, hi);
    if (sub == 0) scales[v] = s;
  }
}

}  // namespace

hipError_t launch_store(const uint16_t* x, int64_t n, const int32_t* pos, const int64_t* slots,
                        const KCache& c, uint32_t flags, float eps, float rope_base, int rope_dim,
                        float* dbg, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 3) / 4)), block(256);
  if (c.dtype == 2)
    hipLaunchKernelGGL(index_k_store_kernel<true>, grid, block, 0, s, x, n, pos, slots, c.base,
                       c.block_size, c.num_blocks, flags, eps, rope_base, rope_dim, dbg);
  else
    hipLaunchKernelGGL(index_k_store_kernel<false>, grid, block, 0, s, x, n, pos, slots, c.base,
                       c.block_size, c.num_blocks, flags, eps, rope_base, rope_dim, dbg);
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
