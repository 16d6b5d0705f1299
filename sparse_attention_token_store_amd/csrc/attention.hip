// Sparse decode attention over the indexer's selections: every query head of a row
// attends over the KV states of the row's selected slots only,
//     o_h = sum_j softmax_j(scale * q_h . kv[s_j]) kv[s_j],   lse_h = log sum_j exp(...)
// with one 512-dim compressed KV state per token serving as key and value (the
// consumer of the top-k: ROCm/ATOM issue 1507, "How it was isolated", decode
// attention after the logical -> physical translation; "The Pivot: A Single Edit
// ...", "Assumptions and Input Knowledge": head_dim 512 for the main KV).
//
// Design for gfx950:
//  - A workgroup takes one row, one run of its slot list (a split) and up to 64
//    heads, one wavefront per 16 heads.  The run is streamed in stages of 32 KV rows
//    (32 KB of bf16) that LDS DMA (global_load_lds, one 1 KB row per wavefront
//    instruction, non-temporal: every row is read once) copies into a double-buffered
//    LDS stage, so the next stage is in flight while the current one is scored.
//  - Scores run transposed, S^T = K . Q^T, on v_mfma_f32_16x16x32_bf16: A is 16 KV
//    rows x 32 dims from LDS, B is the wavefront's 16 query heads, held in registers
//    for the whole run.  The accumulator then holds, in lane l, head l % 16 and keys
//    4*(l/16) + i of each 16-key tile: the online softmax of a head is in-lane plus
//    one exchange over the four lane groups, and the probabilities are already laid
//    out as the B operand of the second product.
//  - O^T = V^T . P^T on the same MFMA: B is P^T from the score registers (bf16), A is
//    V^T read from the staged rows, four dimensions per 8-byte read (A tile a, row i
//    <-> dimension 64*q + 4*i + a), so one read feeds four output tiles.  A lane's
//    output accumulators all belong to its own head, so the per-head rescaling of the
//    online softmax is a multiply by a lane-local factor.
//  - Stage rows are padded to 1056 bytes and the 16-byte chunks of rows 8..15 of each
//    16 are swapped in pairs, so both read patterns hit distinct banks.
//  - A row's split results (unnormalised output, running max and sum) are merged by
//    a second kernel in a fixed order; with one split the first kernel writes the
//    result directly.  Listed slots < 0 are padding; a slot >= num_slots makes the
//    row's output NaN without being read.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kKvDim = 512;
constexpr int kStageKeys = 32;
constexpr int kPitch = 1056;                        // bytes per staged KV row
constexpr int kStageBytes = kStageKeys * kPitch;    // 33,792
constexpr int kRing = 3;                            // stages: two in flight, one scored
constexpr int kMaxSplitKeys = 2048;                 // slots per split (its slot table in LDS)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t as_b8(uint4 v) {
  union {
    uint4 u;
    bf16x8_t b;
  } x;
  x.u = v;
  return x.b;
}

// byte offset, within the staged row `r`, of 16-byte chunk `c` (chunks of rows whose
// bit 3 is set are swapped in pairs)
__device__ __forceinline__ int chunk_off(int r, int c) { return (c ^ ((r >> 3) & 1)) << 4; }

// Issue the LDS DMA of one stage: wavefront w copies rows w, w + 4, ... of the 32.
// `slot_lane` holds, in lane i < 32, the readable slot of row i.  A row is one
// instruction: lane l loads the 16-byte chunk that belongs at position l of the
// staged row (non-temporal: each KV row is read once).
__device__ __forceinline__ void issue_stage(uint32_t stage_lds, const uint8_t* kv, int slot_lane, int wave,
                                            int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int j = 0; j < kStageKeys / 4; ++j) {
    const int r = wave + 4 * j;
    const int64_t slot = __builtin_amdgcn_readlane(slot_lane, r);
    const int c = lane ^ ((r >> 3) & 1);  // the global chunk for LDS position `lane`
    __builtin_amdgcn_global_load_lds(kv + slot * (kKvDim * 2) + c * 16,
                                     (lds_void*)(uintptr_t)(stage_lds + r * kPitch), 16, 0, 2);
  }
}

template <int DP>  // the output dims of a head group are split over DP wavefronts
__global__ __launch_bounds__(256) void attn_split_kernel(
    const uint16_t* __restrict__ q, int heads, const uint8_t* __restrict__ kv, int64_t num_slots,
    const int64_t* __restrict__ slots, int64_t ld, int k, float scale_log2, int keys_per_split,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int HG = 4 / DP;        // head groups of 16 per workgroup
  constexpr int NQ = 8 / DP;        // 64-dim output groups per wavefront
  __shared__ __attribute__((aligned(16))) uint8_t stage[kRing * kStageBytes];
  __shared__ int32_t sl[kMaxSplitKeys];  // the run's slots: >= 0 readable, -1 padding, -2 out of range
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, r = blockIdx.y;
  const int hg = wave % HG, dp = wave / HG;
  const int h0 = blockIdx.z * (16 * HG) + 16 * hg;    // this wavefront's first head
  const int qd0 = dp * NQ;                             // its first 64-dim output group
  const int nsplit = gridDim.x;
  const int k0 = split * keys_per_split;
  const int k1 = min(k, k0 + keys_per_split);
  const int n = max(0, k1 - k0);
  const int nst = (n + kStageKeys - 1) / kStageKeys;
  const int hl = lane & 15, g = lane >> 4;
  const uint32_t slb = (uint32_t)(uintptr_t)sl;
  const uint32_t stb = (uint32_t)(uintptr_t)stage;

  // the run's slot list, classified once (rows past the run are padding)
  for (int i = threadIdx.x; i < nst * kStageKeys; i += 256) {
    const int64_t s = i < n ? slots[(int64_t)r * ld + k0 + i] : -1;
    sl[i] = s < 0 ? -1 : (s >= num_slots ? -2 : (int32_t)s);
  }
  // B operand of the scores: head h0 + hl, dims 32*s + 8*g .. +7, for s < 16
  bf16x8_t qb[16];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)r * heads + h0 + hl) * kKvDim);
#pragma unroll
    for (int s = 0; s < 16; ++s) qb[s] = as_b8(qp[4 * s + g]);
  }
  __syncthreads();

  // entry (lane & 31) of stage st's slots, and the ballots of its padding and
  // out-of-range rows (read with an explicit wait: the compiler would otherwise wait
  // for every LDS DMA in flight before an LDS read)
  auto stage_slot = [&](int st, uint64_t* pad, uint64_t* bad) {
    int32_t s;
    __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(s)
                     : "v"(slb + 4u * (uint32_t)(st * kStageKeys + (lane & 31)))
                     : "memory");
    *pad = __ballot(s == -1) & 0xFFFFFFFFull;
    *bad = __ballot(s == -2) & 0xFFFFFFFFull;
    return s < 0 ? 0 : s;
  };

  f32x4_t acc_o[4 * NQ];  // O^T: output group qd0 + qq, tile a: index 4*qq + a
#pragma unroll
  for (int t = 0; t < 4 * NQ; ++t) acc_o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max (log2 domain) of this lane's head
  float l = 0.0f;       // this lane's share of the running sum (keys 4g + i of every tile)
  bool row_bad = false;

  // stages 0 and 1 go in flight before the loop; (pad0, bad0) belong to the stage
  // being scored, (pad1, bad1) to the next one
  uint64_t pad0 = 0, bad0 = 0, pad1 = 0, bad1 = 0;
  if (nst > 0) issue_stage(stb, kv, stage_slot(0, &pad0, &bad0), wave, lane);
  if (nst > 1) issue_stage(stb + kStageBytes, kv, stage_slot(1, &pad1, &bad1), wave, lane);

  for (int st = 0; st < nst; ++st) {
    // this wavefront's rows of stage st have landed (stage st + 1's may still be in
    // flight); after the barrier every wavefront's have, and every wavefront is done
    // with stage st - 1, whose buffer takes stage st + 2
    if (st + 1 < nst)
      __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kStageKeys / 4) : "memory");
    else
      __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    uint64_t pad2 = 0, bad2 = 0;
    if (st + 2 < nst)
      issue_stage(stb + ((st + 2) % kRing) * kStageBytes, kv, stage_slot(st + 2, &pad2, &bad2), wave, lane);
    const uint32_t sb = stb + (st % kRing) * kStageBytes;
    const uint64_t mask_cur = pad0 | bad0;
    row_bad = row_bad || bad0 != 0;

    // ---- scores S^T for 32 keys (two 16-key tiles) x 16 heads.  The 16-byte chunk
    // 4s + g of row 16t + hl sits at (4s + (g ^ sw)) * 16, sw = bit 3 of the row: a
    // fixed row address plus the immediate offset 64 * s.
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    uint32_t kbase[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 16 * t + hl;
      kbase[t] = sb + row * kPitch + ((g ^ ((row >> 3) & 1)) << 4);
    }
#pragma unroll
    for (int s4 = 0; s4 < 16; s4 += 2) {
      uint4 a[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        __asm__ volatile(
            "ds_read_b128 %0, %2 offset:%3\n\t"
            "ds_read_b128 %1, %2 offset:%4\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a[t][0]), "=&v"(a[t][1])
            : "v"(kbase[t]), "n"(64 * s4), "n"(64 * (s4 + 1))
            : "memory");
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(a[t][j]), qb[s4 + j], sacc[t], 0, 0, 0);
    }

    // ---- online softmax of head hl over this stage's keys 16t + 4g + i
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * t + 4 * g + i;
        const bool masked = (mask_cur >> key) & 1;
        const float v = masked ? -INFINITY : sacc[t][i] * scale_log2;
        sv[4 * t + i] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m, cmax);
    // (a head with nothing visible yet keeps m = -inf and all-zero state)
    const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m - m_new);
    const float msub = m_new == -INFINITY ? 0.0f : m_new;
    float psum = 0.0f;
    bf16x8_t pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2f(sv[j] - msub);
      psum += p;
      pb[j] = (__bf16)p;
    }
    l = l * alpha + psum;
    m = m_new;
    if (__ballot(alpha != 1.0f)) {  // the running max moved for some head
#pragma unroll
      for (int t = 0; t < 4 * NQ; ++t) acc_o[t] *= alpha;
    }

    // ---- O^T += V^T . P^T; k-slot j of lane group g is key 4g + j (j < 4) or
    // 16 + 4g + j - 4 (j >= 4), as in the score accumulator.  Dims 64*qd + 4*hl .. +3
    // of row `row` sit at byte 128*qd + (((hl >> 1) ^ sw) << 4) + 8*(hl & 1): a fixed
    // row address plus the immediate offset 128 * (qd - qd0).
    uint32_t vbase[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
      vbase[j] = sb + row * kPitch + 128 * qd0 + (((hl >> 1) ^ ((row >> 3) & 1)) << 4) + 8 * (hl & 1);
    }
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      uint2 v[8];
      __asm__ volatile(
          "ds_read_b64 %0, %8 offset:%16\n\t"
          "ds_read_b64 %1, %9 offset:%16\n\t"
          "ds_read_b64 %2, %10 offset:%16\n\t"
          "ds_read_b64 %3, %11 offset:%16\n\t"
          "ds_read_b64 %4, %12 offset:%16\n\t"
          "ds_read_b64 %5, %13 offset:%16\n\t"
          "ds_read_b64 %6, %14 offset:%16\n\t"
          "ds_read_b64 %7, %15 offset:%16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
            "=&v"(v[7])
          : "v"(vbase[0]), "v"(vbase[1]), "v"(vbase[2]), "v"(vbase[3]), "v"(vbase[4]), "v"(vbase[5]),
            "v"(vbase[6]), "v"(vbase[7]), "n"(128 * qq)
          : "memory");
      // tile a takes bf16 element a of each read: dims 64*qd + 4*hl + a
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        union {
          uint32_t w[4];
          bf16x8_t b;
        } op;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t lo = (a < 2 ? v[2 * jj].x : v[2 * jj].y) >> (16 * (a & 1));
          const uint32_t hi = (a < 2 ? v[2 * jj + 1].x : v[2 * jj + 1].y) >> (16 * (a & 1));
          op.w[jj] = (lo & 0xFFFFu) | (hi << 16);
        }
        acc_o[4 * qq + a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.b, pb, acc_o[4 * qq + a], 0, 0, 0);
      }
    }
    pad0 = pad1;
    bad0 = bad1;
    pad1 = pad2;
    bad1 = bad2;
  }

  // ---- the head's full sum over the four lane groups
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int h = h0 + hl;
  // lane (hl, g) holds O^T rows 4g + i of tile a of group qd: dims 64*qd + 4*(4g + i) + a
  // = 64*qd + 16*g + 4*i + a, i.e. 16 consecutive dims per group qd
  if (nsplit == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float nanv = __builtin_nanf("");
    float* orow = out + ((int64_t)r * heads + h) * kKvDim;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 v4;
        v4.x = row_bad ? nanv : acc_o[4 * qq + 0][i] * inv;
        v4.y = row_bad ? nanv : acc_o[4 * qq + 1][i] * inv;
        v4.z = row_bad ? nanv : acc_o[4 * qq + 2][i] * inv;
        v4.w = row_bad ? nanv : acc_o[4 * qq + 3][i] * inv;
        *reinterpret_cast<float4*>(orow + 64 * (qd0 + qq) + 16 * g + 4 * i) = v4;
      }
    }
    if (lse && g == 0 && dp == 0)
      lse[(int64_t)r * heads + h] = row_bad ? nanv : (l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY);
    return;
  }
  // split results: unnormalised O, and (max, sum) in the log2 domain; a bad slot in
  // the run makes the sum NaN, which the merge carries into the row's output
  float* po = part_o + (((int64_t)r * nsplit + split) * heads + h) * kKvDim;
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 v4;
      v4.x = acc_o[4 * qq + 0][i];
      v4.y = acc_o[4 * qq + 1][i];
      v4.z = acc_o[4 * qq + 2][i];
      v4.w = acc_o[4 * qq + 3][i];
      *reinterpret_cast<float4*>(po + 64 * (qd0 + qq) + 16 * g + 4 * i) = v4;
    }
  if (g == 0 && dp == 0) {
    float* pm = part_ml + (((int64_t)r * nsplit + split) * heads + h) * 2;
    pm[0] = m;
    pm[1] = row_bad ? __builtin_nanf("") : l;
  }
}

// Merge of a row's split results, in split order: one workgroup per (row, head),
// one thread per two dims.
__global__ __launch_bounds__(256) void attn_merge_kernel(int heads, int nsplit, const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  const int h = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  float M = -INFINITY;
  bool bad = false;
  for (int j = 0; j < nsplit; ++j) {
    const float* pm = part_ml + (((int64_t)r * nsplit + j) * heads + h) * 2;
    M = fmaxf(M, pm[0]);
    bad = bad || (pm[1] != pm[1]);
  }
  float z = 0.0f, o0 = 0.0f, o1 = 0.0f;
  if (M != -INFINITY) {
    for (int j = 0; j < nsplit; ++j) {
      const float* pm = part_ml + (((int64_t)r * nsplit + j) * heads + h) * 2;
      const float w = exp2f(pm[0] - M);  // 0 for a split that saw nothing
      const float2 o = reinterpret_cast<const float2*>(part_o + (((int64_t)r * nsplit + j) * heads + h) * kKvDim)[t];
      z += w * pm[1];
      o0 += w * o.x;
      o1 += w * o.y;
    }
  }
  const float inv = z > 0.0f ? 1.0f / z : 0.0f;
  float2 res = make_float2(o0 * inv, o1 * inv);
  if (bad) res = make_float2(__builtin_nanf(""), __builtin_nanf(""));
  reinterpret_cast<float2*>(out + ((int64_t)r * heads + h) * kKvDim)[t] = res;
  if (lse && t == 0)
    lse[(int64_t)r * heads + h] = bad ? __builtin_nanf("") : (z > 0.0f ? (M + __log2f(z)) * kLn2 : -INFINITY);
}

struct SplitPlan {
  int splits, keys_per_split;
};

// Splits of each row's list: about one workgroup per CU (the LDS ring allows one),
// at least two stages per split, split results (2 x 4 B x heads x 512 per split,
// written and read back) at most half the KV bytes they stand for (k x 1 KB), and
// no split longer than its LDS slot table.
SplitPlan plan_splits(int rows, int k, int heads) {
  if (k <= 0) return SplitPlan{1, kStageKeys};
  const int hgroups = (heads + 63) / 64;
  const int stages = (k + kStageKeys - 1) / kStageKeys;
  int s = (256 + rows * hgroups - 1) / (rows * hgroups);
  s = std::min(s, std::max(1, stages / 2));
  s = std::min(s, std::max(1, k / (8 * heads)));
  s = std::max(s, (stages + kMaxSplitKeys / kStageKeys - 1) / (kMaxSplitKeys / kStageKeys));
  s = std::max(s, 1);
  const int per = ((stages + s - 1) / s) * kStageKeys;
  return SplitPlan{(k + per - 1) / per, per};
}

}  // namespace

size_t attention_ws_bytes(int rows, int k, int heads) {
  const SplitPlan p = plan_splits(rows, k, heads);
  if (p.splits <= 1) return 0;
  return (size_t)rows * p.splits * heads * (kKvDim + 2) * 4;
}

hipError_t launch_attention(const uint16_t* q, int heads, const uint8_t* kv, int64_t num_slots, const int64_t* slots,
                            int64_t ld, int k, int rows, float scale, float* out, float* lse, void* ws,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const SplitPlan p = plan_splits(rows, k, heads);
  float* part_o = static_cast<float*>(ws);
  float* part_ml = p.splits > 1 ? part_o + (size_t)rows * p.splits * heads * kKvDim : nullptr;
  const int wg_heads = heads < 64 ? heads : 64;
  const dim3 grid((unsigned)p.splits, (unsigned)rows, (unsigned)(heads / wg_heads));
  const float scale_log2 = scale * kLog2e;
  switch (64 / wg_heads) {  // dim parts per head group
#define DSA_ATTN_CASE(DP)                                                                                    \
  case DP:                                                                                                   \
    hipLaunchKernelGGL(attn_split_kernel<DP>, grid, dim3(256), 0, s, q, heads, kv, num_slots, slots, ld, k, \
                       scale_log2, p.keys_per_split, out, lse, part_o, part_ml);                             \
    break;
    DSA_ATTN_CASE(1)
    DSA_ATTN_CASE(2)
    DSA_ATTN_CASE(4)
#undef DSA_ATTN_CASE
    default:
      return hipErrorInvalidValue;
  }
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)heads, (unsigned)rows), dim3(256), 0, s, heads, p.splits,
                       part_o, part_ml, out, lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
