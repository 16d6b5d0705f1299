// Sparse decode attention over the indexer's selections: every query head of a row
// attends over the KV states of the row's selected slots only,
//     o_h = sum_j softmax_j(scale * q_h . kv[s_j]) kv[s_j],   lse_h = log sum_j exp(...)
// with one 512-dim compressed KV state per token serving as key and value (the
// consumer of the top-k: ROCm/ATOM issue 1507, "How it was isolated", decode
// attention after the logical -> physical translation; "The Pivot: A Single Edit
// ...", "Assumptions and Input Knowledge": head_dim 512 for the main KV).
//
// Design for gfx950:
//  - A workgroup of four wavefronts takes one row, one run of its slot list (a
//    split) and 16 or 32 heads: the wavefronts of a 16-head group split its 512
//    output dims 4 or 2 ways.  With more than 32 heads, further workgroups take the
//    further 32-head groups; each reads the run's KV rows again (mostly from L2),
//    whereas a 64-head workgroup held all 512 output dims of its 16 heads in each
//    wavefront's registers, one wavefront per SIMD, and was slower (27.2 against
//    24.2 us for 32 rows x top-512 with 64 heads).  The run is streamed
//    in stages of 32 KV rows (32 KB of bf16) that LDS DMA (global_load_lds, one 1 KB
//    row per wavefront instruction, non-temporal: every row is read once) copies into
//    a ring of three LDS stages, two in flight while the third is scored.
//  - Scores run transposed, S^T = K . Q^T, on v_mfma_f32_16x16x32_bf16: A is 16 KV
//    rows x 32 dims from LDS, B is the wavefront's 16 query heads, held in registers
//    for the whole run.  The accumulator then holds, in lane l, head l % 16 and keys
//    4*(l/16) + i of each 16-key tile: the online softmax of a head is in-lane plus
//    one exchange over the four lane groups, and the probabilities are already laid
//    out as the B operand of the second product.
//  - O^T = V^T . P^T on the same MFMA: B is P^T from the score registers (bf16), A is
//    V^T read from the staged rows with gfx950's transposing LDS read
//    (ds_read_b64_tr_b16), two reads per 16-dim tile and no repacking.  A lane's
//    output accumulators all belong to its own head, so the per-head rescaling of the
//    online softmax is a multiply by a lane-local factor.
//  - Staged rows are 1 KB, with 16-byte chunk c of row r at position c ^ (r & 15):
//    both read patterns (16 rows at one chunk; 4 rows x 32 bytes) hit distinct banks.
//  - The running max of the online softmax only moves when a stage exceeds it by more
//    than 2^8, so the accumulators are rescaled rarely.
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
constexpr int kRowBytes = kKvDim * 2;               // one bf16 KV row, staged unpadded
constexpr int kStageBytes = kStageKeys * kRowBytes; // 32 KB
constexpr int kMaxSplitKeys = 2048;                 // slots per split (its slot table in LDS)
constexpr float kLazy = 8.0f;                       // log2 headroom of the running max
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

// Issue the LDS DMA of one stage: wavefront w copies rows w, w + 4, ... of the 32.
// `slot_lane` holds, in lane i < 32, the readable slot of row i.  A row is one
// instruction: lane l writes 16-byte position l of the staged row, which holds the
// row's chunk l ^ (r & 15) (non-temporal: each KV row is read once).
__device__ __forceinline__ void issue_stage(uint32_t stage_lds, const uint8_t* kv, int slot_lane, int wave,
                                            int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int j = 0; j < kStageKeys / 4; ++j) {
    const int r = wave + 4 * j;
    const int64_t slot = __builtin_amdgcn_readlane(slot_lane, r);
    __builtin_amdgcn_global_load_lds(kv + slot * kRowBytes + ((lane ^ (r & 15)) << 4),
                                     (lds_void*)(uintptr_t)(stage_lds + r * kRowBytes), 16, 0, 2);
  }
}

template <int DP, int RING>  // output dims of a head group split over DP wavefronts;
                             // RING LDS stages (RING - 1 in flight)
__global__ __launch_bounds__(256) void attn_split_kernel(
    const uint16_t* __restrict__ q, int heads, const uint8_t* __restrict__ kv, int64_t num_slots,
    const int64_t* __restrict__ slots, int64_t ld, int k, float scale_log2, int keys_per_split,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int HG = 4 / DP;        // head groups of 16 per workgroup
  constexpr int NT = 32 / DP;       // 16-dim output tiles per wavefront
  __shared__ __attribute__((aligned(16))) uint8_t stage[RING * kStageBytes];
  __shared__ int32_t sl[kMaxSplitKeys];  // the run's slots: >= 0 readable, -1 padding, -2 out of range
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, r = blockIdx.y;
  const int hg = wave % HG, dp = wave / HG;
  const int h0 = blockIdx.z * (16 * HG) + 16 * hg;    // this wavefront's first head
  const int t0 = dp * NT;                              // its first 16-dim output tile
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

  // Stage addresses.  Chunk c (16 bytes) of staged row r sits at position c ^ (r & 15)
  // of its 1 KB row.
  //  - Score operand of lane (hl, g), k-step s: chunk 4s + g of rows hl and 16 + hl
  //    (the same r & 15): position ((4s + g) ^ hl) = (4*(s & 3) + g) ^ hl + 16*(s >> 2),
  //    so four row addresses (s & 3) and the immediate offset 256*(s >> 2) (+16 KB for
  //    the second tile) reach every k-step.
  //  - Transposed read of tile T (dims 16T .. 16T+15) for lane (hl, g): row ra = 4g +
  //    hl/4 (and 16 + ra), bytes 8*(hl % 4) of the tile's 32: chunk 2T + ((hl >> 1) & 1)
  //    at position (2*(T & 7) + ((hl >> 1) & 1)) ^ (ra & 15) + 16*(T >> 3): eight row
  //    addresses (T & 7) and the immediate offset 256*(T >> 3).
  uint32_t koff[4], voff[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = hl * kRowBytes + (((4 * j + g) ^ hl) << 4);
  {
    const int ra = 4 * g + (hl >> 2);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      voff[j] = ra * kRowBytes + (((2 * j + ((hl >> 1) & 1)) ^ (ra & 15)) << 4) + 8 * (hl & 1);
  }

  f32x4_t acc_o[NT];  // O^T tiles: dims 16*(t0 + tt) .. +15 x 16 heads
#pragma unroll
  for (int t = 0; t < NT; ++t) acc_o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Running max (log2 domain) of this lane's head.  It is raised only when a stage's
  // scores exceed it by more than kLazy (so probabilities stay below 2^kLazy and the
  // accumulators are rescaled rarely); the sums use the same reference, so the
  // result does not depend on when it moved.
  float m = -INFINITY;
  float l = 0.0f;       // this lane's share of the running sum (keys 4g + i of every tile)
  bool row_bad = false;

  // RING - 1 stages go in flight before the loop; (pad[j], bad[j]) belong to stage st + j
  uint64_t pad0 = 0, bad0 = 0, pad1 = 0, bad1 = 0;
  if (nst > 0) issue_stage(stb, kv, stage_slot(0, &pad0, &bad0), wave, lane);
  if (RING > 2 && nst > 1) issue_stage(stb + kStageBytes, kv, stage_slot(1, &pad1, &bad1), wave, lane);

  for (int st = 0; st < nst; ++st) {
    // this wavefront's rows of stage st have landed (with RING = 3, stage st + 1's
    // may still be in flight); after the barrier every wavefront's have, and every
    // wavefront is done with stage st - 1, whose buffer is refilled next
    if (RING > 2 && st + 1 < nst)
      __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kStageKeys / 4) : "memory");
    else
      __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    uint64_t padn = 0, badn = 0;
    const int nx = st + RING - 1;  // the stage issued now
    if (nx < nst) issue_stage(stb + (nx % RING) * kStageBytes, kv, stage_slot(nx, &padn, &badn), wave, lane);
    if (RING == 2) {  // (stage st + 1's masks come with its issue)
      pad1 = padn;
      bad1 = badn;
    }
    const uint32_t sb = stb + (st % RING) * kStageBytes;
    const uint64_t mask_cur = pad0 | bad0;
    row_bad = row_bad || bad0 != 0;

    // ---- scores S^T for 32 keys (two 16-key tiles) x 16 heads: eight reads per wait
    // (four k-steps of both tiles); two accumulators per tile (even and odd k-steps)
    // keep four independent MFMA chains
    f32x4_t sacc[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) sacc[t][0] = sacc[t][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 16; s4 += 4) {
      uint4 a0, a1, a2, a3, b0, b1, b2, b3;
      __asm__ volatile(
          "ds_read_b128 %0, %8 offset:%12\n\t"
          "ds_read_b128 %1, %9 offset:%12\n\t"
          "ds_read_b128 %2, %10 offset:%12\n\t"
          "ds_read_b128 %3, %11 offset:%12\n\t"
          "ds_read_b128 %4, %8 offset:%13\n\t"
          "ds_read_b128 %5, %9 offset:%13\n\t"
          "ds_read_b128 %6, %10 offset:%13\n\t"
          "ds_read_b128 %7, %11 offset:%13\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
          : "v"(sb + koff[0]), "v"(sb + koff[1]), "v"(sb + koff[2]), "v"(sb + koff[3]), "n"(64 * s4),
            "n"(64 * s4 + 16 * kRowBytes)
          : "memory");
      sacc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(a0), qb[s4], sacc[0][0], 0, 0, 0);
      sacc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(b0), qb[s4], sacc[1][0], 0, 0, 0);
      sacc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(a1), qb[s4 + 1], sacc[0][1], 0, 0, 0);
      sacc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(b1), qb[s4 + 1], sacc[1][1], 0, 0, 0);
      sacc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(a2), qb[s4 + 2], sacc[0][0], 0, 0, 0);
      sacc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(b2), qb[s4 + 2], sacc[1][0], 0, 0, 0);
      sacc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(a3), qb[s4 + 3], sacc[0][1], 0, 0, 0);
      sacc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(b3), qb[s4 + 3], sacc[1][1], 0, 0, 0);
    }
    const f32x4_t sacc_t[2] = {sacc[0][0] + sacc[0][1], sacc[1][0] + sacc[1][1]};

    // ---- online softmax of head hl over this stage's keys 16t + 4g + i
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * t + 4 * g + i;
        const bool masked = (mask_cur >> key) & 1;
        const float v = masked ? -INFINITY : sacc_t[t][i] * scale_log2;
        sv[4 * t + i] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    if (cmax > m + kLazy) {  // (also the first visible key: m = -inf)
      const float alpha = m == -INFINITY ? 0.0f : exp2f(m - cmax);
      m = cmax;
      l *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc_o[t] *= alpha;
    }
    const float msub = m == -INFINITY ? 0.0f : m;  // (nothing visible yet: all p are 0)
    float psum = 0.0f;
    bf16x8_t pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2f(sv[j] - msub);
      psum += p;
      pb[j] = (__bf16)p;
    }
    l += psum;

    // ---- O^T += V^T . P^T.  A is V^T, read transposed with ds_read_b64_tr_b16: lane
    // i of each 16-lane group receives column i of the four rows its group addresses
    // (lane x addresses row x/4, columns 4*(x%4) .. +3).  Two reads give lane (hl, g)
    // dim 16*T + hl of keys 4g .. 4g+3 and 16+4g .. 16+4g+3: k-slots j < 4 and j >= 4,
    // the key order of P^T.
#pragma unroll
    for (int t4 = 0; t4 < NT; t4 += 4) {
      // tiles T = t0 + t4 .. +3: t0 is a multiple of 8, so T & 7 = (t4 & 7) + i, known
      // at compile time, and T >> 3 is the same for all four
      uint2 x0, x1, x2, x3, y0, y1, y2, y3;
      const uint32_t vb = sb + 256 * ((t0 + t4) >> 3);
      const int j0 = t4 & 7;
      __asm__ volatile(
          "ds_read_b64_tr_b16 %0, %8\n\t"
          "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
          "ds_read_b64_tr_b16 %2, %9\n\t"
          "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
          "ds_read_b64_tr_b16 %4, %10\n\t"
          "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
          "ds_read_b64_tr_b16 %6, %11\n\t"
          "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x0), "=&v"(y0), "=&v"(x1), "=&v"(y1), "=&v"(x2), "=&v"(y2), "=&v"(x3), "=&v"(y3)
          : "v"(vb + voff[j0]), "v"(vb + voff[j0 + 1]), "v"(vb + voff[j0 + 2]), "v"(vb + voff[j0 + 3]),
            "n"(16 * kRowBytes)
          : "memory");
      acc_o[t4 + 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(make_uint4(x0.x, x0.y, y0.x, y0.y)), pb,
                                                              acc_o[t4 + 0], 0, 0, 0);
      acc_o[t4 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(make_uint4(x1.x, x1.y, y1.x, y1.y)), pb,
                                                              acc_o[t4 + 1], 0, 0, 0);
      acc_o[t4 + 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(make_uint4(x2.x, x2.y, y2.x, y2.y)), pb,
                                                              acc_o[t4 + 2], 0, 0, 0);
      acc_o[t4 + 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(make_uint4(x3.x, x3.y, y3.x, y3.y)), pb,
                                                              acc_o[t4 + 3], 0, 0, 0);
    }
    pad0 = pad1;
    bad0 = bad1;
    if (RING > 2) {
      pad1 = padn;
      bad1 = badn;
    }
  }

  // ---- the head's full sum over the four lane groups
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int h = h0 + hl;
  // lane (hl, g) holds O^T rows 4g .. 4g+3 of tile tt: dims 16*(t0 + tt) + 4g .. +3
  if (nsplit == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float nanv = __builtin_nanf("");
    float* orow = out + ((int64_t)r * heads + h) * kKvDim + 16 * t0 + 4 * g;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      float4 v4;
      v4.x = row_bad ? nanv : acc_o[tt][0] * inv;
      v4.y = row_bad ? nanv : acc_o[tt][1] * inv;
      v4.z = row_bad ? nanv : acc_o[tt][2] * inv;
      v4.w = row_bad ? nanv : acc_o[tt][3] * inv;
      *reinterpret_cast<float4*>(orow + 16 * tt) = v4;
    }
    if (lse && g == 0 && dp == 0)
      lse[(int64_t)r * heads + h] = row_bad ? nanv : (l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY);
    return;
  }
  // split results: unnormalised O, and (max, sum) in the log2 domain; a bad slot in
  // the run makes the sum NaN, which the merge carries into the row's output
  float* po = part_o + (((int64_t)r * nsplit + split) * heads + h) * kKvDim + 16 * t0 + 4 * g;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
    *reinterpret_cast<float4*>(po + 16 * tt) = make_float4(acc_o[tt][0], acc_o[tt][1], acc_o[tt][2], acc_o[tt][3]);
  if (g == 0 && dp == 0) {
    float* pm = part_ml + (((int64_t)r * nsplit + split) * heads + h) * 2;
    pm[0] = m;
    pm[1] = row_bad ? __builtin_nanf("") : l;
  }
}

// Merge of a row's split results, in split order: one workgroup per (row, 4 heads),
// thread t takes head 4*blockIdx.x + t/64 and dims 8*(t%64) .. +7.  The splits are
// folded in one pass with a running maximum (the output and sum rescaled when it
// moves), eight at a time with all eight splits' loads issued before the first is
// used.
__global__ __launch_bounds__(256) void attn_merge_kernel(int heads, int nsplit, const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  constexpr int kBatch = 8;
  const int t = threadIdx.x, r = blockIdx.y;
  const int h = 4 * blockIdx.x + (t >> 6), d0 = 8 * (t & 63);
  float M = -INFINITY, z = 0.0f;
  float4 o0 = make_float4(0.f, 0.f, 0.f, 0.f), o1 = o0;
  bool bad = false;
  for (int j0 = 0; j0 < nsplit; j0 += kBatch) {
    float2 ml[kBatch];
    float4 a[kBatch], b[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {  // (past the last split: the last split again, unused)
      const int64_t base = ((int64_t)r * nsplit + min(j0 + i, nsplit - 1)) * heads + h;
      ml[i] = *reinterpret_cast<const float2*>(part_ml + base * 2);
      const float4* po = reinterpret_cast<const float4*>(part_o + base * kKvDim + d0);
      a[i] = po[0];
      b[i] = po[1];
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (j0 + i >= nsplit) break;
      bad = bad || (ml[i].y != ml[i].y);
      if (ml[i].x == -INFINITY) continue;  // a split that saw nothing
      const float Mn = fmaxf(M, ml[i].x);
      const float c0 = exp2f(M - Mn), c1 = exp2f(ml[i].x - Mn);  // (M = -inf: c0 = 0)
      z = z * c0 + ml[i].y * c1;
      o0.x = o0.x * c0 + a[i].x * c1; o0.y = o0.y * c0 + a[i].y * c1;
      o0.z = o0.z * c0 + a[i].z * c1; o0.w = o0.w * c0 + a[i].w * c1;
      o1.x = o1.x * c0 + b[i].x * c1; o1.y = o1.y * c0 + b[i].y * c1;
      o1.z = o1.z * c0 + b[i].z * c1; o1.w = o1.w * c0 + b[i].w * c1;
      M = Mn;
    }
  }
  const float inv = z > 0.0f ? 1.0f / z : 0.0f;
  const float nanv = __builtin_nanf("");
  float4 r0 = make_float4(o0.x * inv, o0.y * inv, o0.z * inv, o0.w * inv);
  float4 r1 = make_float4(o1.x * inv, o1.y * inv, o1.z * inv, o1.w * inv);
  if (bad) r0 = r1 = make_float4(nanv, nanv, nanv, nanv);
  float4* op = reinterpret_cast<float4*>(out + ((int64_t)r * heads + h) * kKvDim + d0);
  op[0] = r0;
  op[1] = r1;
  if (lse && (t & 63) == 0)
    lse[(int64_t)r * heads + h] = bad ? nanv : (z > 0.0f ? (M + __log2f(z)) * kLn2 : -INFINITY);
}

struct SplitPlan {
  int splits, keys_per_split;
};

// Splits of each row's list: about one workgroup per CU, at least two stages per
// split, split results (2 x 4 B x heads x 512 per split, written and read back) at
// most twice the KV bytes they stand for (k x 1 KB; a workgroup's stages are
// latency-bound, so spreading a row over more CUs pays for that traffic), and no
// split longer than its LDS slot table.
SplitPlan plan_splits(int rows, int k, int heads) {
  if (k <= 0 || rows <= 0) return SplitPlan{1, kStageKeys};  // nothing to split
  const int hgroups = (heads + 31) / 32;
  const int stages = (k + kStageKeys - 1) / kStageKeys;
  int s = (256 + rows * hgroups - 1) / (rows * hgroups);
  s = std::min(s, std::max(1, stages / 2));
  s = std::min(s, std::max(1, k / (2 * heads)));
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
  const int wg_heads = heads < 32 ? heads : 32;
  const dim3 grid((unsigned)p.splits, (unsigned)rows, (unsigned)(heads / wg_heads));
  const float scale_log2 = scale * kLog2e;
  switch (64 / wg_heads) {  // dim parts per head group
#define DSA_ATTN_CASE(DP, RING)                                                                            \
  case DP:                                                                                                 \
    hipLaunchKernelGGL((attn_split_kernel<DP, RING>), grid, dim3(256), 0, s, q, heads, kv, num_slots, slots, \
                       ld, k, scale_log2, p.keys_per_split, out, lse, part_o, part_ml);                     \
    break;
    DSA_ATTN_CASE(2, 3)   // 104 KB of LDS: one workgroup per CU, two stages in flight
    DSA_ATTN_CASE(4, 2)   // 72 KB: two workgroups per CU, one stage in flight each
#undef DSA_ATTN_CASE
    default:
      return hipErrorInvalidValue;
  }
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(heads / 4), (unsigned)rows), dim3(256), 0, s, heads, p.splits,
                       part_o, part_ml, out, lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
