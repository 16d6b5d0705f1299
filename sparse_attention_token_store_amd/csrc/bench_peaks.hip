// Measurement kernels for the benchmark (built into libdsa_bench.so, not into the
// indexer library): the HBM read rate and the dense MFMA rates this GPU reaches, the
// peaks the indexer kernels are compared with besides the vendor figures, and a
// device-side delay that holds a stream while the host queues the timed steps.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// Holds the stream for `ticks` of the constant-rate wall clock (s_memrealtime).
__global__ void spin_kernel(uint64_t ticks) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

// Streaming read of `n16` 16-byte chunks (a multiple of 8 * threads): each load
// instruction reads consecutive chunks across the grid's threads, eight independent
// loads per step.  The XOR of everything read decides whether one word is written,
// so no load can be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p, uint64_t n16,
                                                          uint32_t* __restrict__ sink) {
  constexpr int kLoads = 8;
  uint32_t acc = 0;
  const uint64_t T = (uint64_t)gridDim.x * 256;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i + (kLoads - 1) * T < n16; i += kLoads * T) {
    u32x4_t v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) v[j] = __builtin_nontemporal_load(p + i + j * T);
    u32x4_t x = v[0];
#pragma unroll
    for (int j = 1; j < kLoads; ++j) x ^= v[j];
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Dense MFMA issue rate: every wavefront runs `iters` rounds of kChains independent
// accumulations (fp8: v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales, the
// prefill scoring instruction; bf16: v_mfma_f32_16x16x32_bf16, the decode one).
constexpr int kChains = 16;
template <bool kFp8>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float seed, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f32x4_t acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (kFp8) {
    const int v = 0x38383838 ^ (lane & 1);
    const i32x8_t a = i32x8_t{v, v, v, v, v, v, v, v};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, acc[j], 0, 0, 0, 127, 0, 127);
  } else {
    bf16x8_t a;
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = (__bf16)(seed + (float)(lane & 3));
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 1.2345f) sink[0] = s;
}

}  // namespace

#define BENCH_API extern "C" __attribute__((visibility("default")))

// Delay the stream by about `microseconds` (device-side; returns at once on the host).
BENCH_API int dsa_bench_spin(double microseconds, void* stream) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return -1;
  const uint64_t ticks = (uint64_t)(microseconds * 1e-3 * (double)khz);
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ticks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Timing events without the system-scope fence a default event performs when it is
// recorded (that fence writes back and invalidates the caches, which both costs
// time between kernels and slows the kernel that follows).  Read only after the
// stream has been synchronised.
BENCH_API void* dsa_bench_event_create(void) {
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}
BENCH_API int dsa_bench_event_record(void* e, void* stream) {
  return hipEventRecord(static_cast<hipEvent_t>(e), static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : -1;
}
BENCH_API float dsa_bench_event_ms(void* a, void* b) {
  float ms = -1.0f;
  if (hipEventElapsedTime(&ms, static_cast<hipEvent_t>(a), static_cast<hipEvent_t>(b)) != hipSuccess) return -1.0f;
  return ms;
}
BENCH_API void dsa_bench_event_destroy(void* e) { (void)hipEventDestroy(static_cast<hipEvent_t>(e)); }

// Read `bytes` (a multiple of 128 * 256 * blocks) from the device buffer `buf` once.
BENCH_API int dsa_bench_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!buf || !sink || blocks < 1 || bytes % (128ull * 256 * (uint64_t)blocks)) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Run the MFMA rate kernel (fp8 = 1: scaled f8f6f4 16x16x128; 0: bf16 16x16x32) on
// `blocks` workgroups of 4 wavefronts; *flops receives the dense FLOP count of the launch.
BENCH_API int dsa_bench_mfma(int fp8, int blocks, int iters, float* sink, double* flops, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return -1;
  const double per = fp8 ? 2.0 * 16 * 16 * 128 : 2.0 * 16 * 16 * 32;
  if (flops) *flops = per * kChains * (double)iters * 4.0 * blocks;
  if (fp8)
    hipLaunchKernelGGL(mfma_rate_kernel<true>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       1.0f, sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<false>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       1.0f, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
