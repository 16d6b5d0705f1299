// Chunked-prefill scoring: many fp8 query rows (per (row, head) e4m3 codes and
// fp32 scale) against the paged fp8 index-K cache,
//     score[r][p] = s_p * sum_h w[r][h] * qs[r][h] * max(0, qc[r][h] . kc[p])
// which equals sum_h w_h max(0, q_h . k_p) on the dequantised values since both
// scales are positive (the pages' fp8_mqa_logits path, ROCm/ATOM issue 1507, "How
// it was isolated" and "Recommended fix": the query is fp8-quantised before scoring).
//
// Design for gfx950:
//  - The (query row, head) pairs form the MFMA M dimension and the keys the N
//    dimension; head_dim 128 is exactly the K of one v_mfma_scale_f32_16x16x128_f8f6f4,
//    so one instruction produces 16 (row, head) logits for 16 keys.  Block scales
//    are 2^0: the real scales are folded into the epilogue.
//  - Workgroup = 8 waves, one query row per wave, 8 consecutive rows of one
//    sequence.  Each wave keeps its row's 64 heads as 4 A tiles in registers.
//  - The 8 waves share the keys through LDS: every 64-key span (8 KB of codes plus
//    256 B of scales) is loaded once per workgroup with one 16-byte chunk per
//    thread, prefetched two spans ahead in registers and written to a double-buffered
//    LDS stage.  Key rows are padded to 144 bytes: 16-byte reads of 16 consecutive
//    keys at the same offset then fall on 16 distinct bank groups (9r mod 16 is a
//    permutation), so the B-operand reads, lane = (key, 32-byte quarter), do not
//    conflict.  About 120 VGPRs per wave: 4 waves per SIMD hide the latency.
//  - Within a wave the next 16-key group's LDS reads and MFMAs are issued before the
//    current group's epilogue, so the matrix core and the VALU overlap.
//  - Keys are split into 8 chunks and workgroup w takes chunk w mod 8.  Workgroups
//    are dispatched to the 8 XCDs round robin, so each XCD's L2 only ever holds its
//    eighth of the keys.
//  - Epilogue per 16-key tile: ReLU, weight by w*qs, in-lane head sum over the 16
//    heads a lane holds, a cross-row permute sum, per-key scale.
//  - A workgroup whose rows read different sequences falls back to per-wave direct
//    loads (correct, slower; chunked prefill never takes it).
#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kSpan = 64;
constexpr int kWavesPf = 8;                 // one query row per wave
constexpr int kThreadsPf = 64 * kWavesPf;
constexpr int kKeyChunks = 8;
constexpr int kRowPitch = 144;                       // padded LDS key row
constexpr int kScaleOff = kSpan * kRowPitch;          // scales after the 64 rows
constexpr int kStage = kScaleOff + kSpan * 4;         // 9472 bytes per staged span

// One thread's share of a span: code chunk tid & 7 of key tid >> 3, and for tid < 16
// the 16 bytes of scales of keys 4*tid .. 4*tid+3.
struct Share {
  uint4 code;
  uint4 scale;
};

template <int BS>
__device__ __forceinline__ void load_share(Share& sh, const uint8_t* cache, int64_t num_blocks,
                                           const int32_t* bt_row, int p_span, int n_max, int tid) {
  const int key = tid >> 3;
  const int c = tid & 7;
  const int pos = p_span + key;
  if (pos < n_max) {
    int phys = bt_row[pos / BS];
    phys = (phys < 0 || phys >= num_blocks) ? 0 : phys;
    sh.code = *reinterpret_cast<const uint4*>(cache + (int64_t)phys * (BS * 132) + (pos % BS) * 128 + c * 16);
  }
  if (tid < 16) {
    const int p4 = p_span + 4 * tid;
    if (p4 < n_max) {
      int phys = bt_row[p4 / BS];
      phys = (phys < 0 || phys >= num_blocks) ? 0 : phys;
      sh.scale = *reinterpret_cast<const uint4*>(cache + (int64_t)phys * (BS * 132) + BS * 128 + (p4 % BS) * 4);
    }
  }
}

__device__ __forceinline__ void store_share(uint8_t* stage, const Share& sh, int tid) {
  *reinterpret_cast<uint4*>(stage + (tid >> 3) * kRowPitch + (tid & 7) * 16) = sh.code;
  if (tid < 16) *reinterpret_cast<uint4*>(stage + kScaleOff + tid * 16) = sh.scale;
}

// B operand of group g for this lane: key 16g + lane%16, code bytes 32*(lane/16) .. +31
__device__ __forceinline__ i32x8_t read_b(const uint8_t* stage, int g, int lane) {
  const uint8_t* p = stage + (16 * g + (lane & 15)) * kRowPitch + 32 * (lane >> 4);
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
__device__ __forceinline__ float read_scale(const uint8_t* stage, int g, int lane) {
  return reinterpret_cast<const float*>(stage + kScaleOff)[16 * g + (lane & 15)];
}

// Epilogue of one 16-key group: the row's score for key 16g + lane%16 (in every
// 16-lane row of the wave).
__device__ __forceinline__ float group_score(const f32x4_t (&acc)[4], const float (&wq)[4][4], float s) {
  float part = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) part = fmaf(wq[mt][v], relu(acc[mt][v]), part);
  return rows4_sum(part) * s + 0.0f;  // +0.0f: a zero score is +0
}

template <int BS>
__global__ __launch_bounds__(kThreadsPf, 2) void score_prefill_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ cache, int64_t num_blocks, const int32_t* __restrict__ block_table,
    int max_blocks, int num_seqs, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, int rows, int max_row_len, float* __restrict__ scores,
    int64_t ld, int chunk_keys, int write_pad) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[2][kStage];
  __shared__ int wg_seq[kWavesPf];
  __shared__ int wg_len[kWavesPf];

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x % kKeyChunks;
  const int tile = blockIdx.x / kKeyChunks;
  const int row = tile * kWavesPf + wave;
  const int k0 = chunk * chunk_keys;
  const int k1 = min(k0 + chunk_keys, max_row_len);

  // this wave's row: length, sequence (-1: no row, -2: sequence out of range)
  const bool in = row < rows;
  const int n = in ? min(max(row_len[row], 0), max_row_len) : 0;
  int seq = in ? row_seq[row] : -1;
  if (in && (seq < 0 || seq >= num_seqs)) seq = -2;
  if (lane == 0) {
    wg_seq[wave] = seq;
    wg_len[wave] = n;
  }
  __syncthreads();
  // one sequence shared by every live row of the workgroup?
  int s0 = -1, n_max = 0;
  bool shared = true;
#pragma unroll
  for (int i = 0; i < kWavesPf; ++i) {
    const int si = wg_seq[i];
    if (si < 0) continue;
    if (s0 < 0) s0 = si;
    shared = shared && si == s0;
    n_max = max(n_max, wg_len[i]);
  }
  if (k0 >= k1) return;  // uniform: an empty key chunk

  float* out = scores + (int64_t)(in ? row : 0) * ld;
  if (seq == -2) {  // a row whose sequence is out of range scores NaN where it sees keys
    for (int p = k0 + lane; p < k1; p += 64) {
      if (p < n) out[p] = __builtin_nanf("");
      else if (write_pad) out[p] = -INFINITY;
    }
  }
  const bool active = seq >= 0;

  // A operands of this row: head 16*mt + lane%16, code bytes 32*(lane/16) .. +31
  i32x8_t qa[4];
  float wq[4][4];  // w * q_scale of the accumulator rows this lane holds
  if (active) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      qa[mt] = *reinterpret_cast<const i32x8_t*>(
          q + ((int64_t)row * 64 + 16 * mt + (lane & 15)) * kHeadDim + 32 * (lane >> 4));
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * mt + 4 * (lane >> 4) + v;
        wq[mt][v] = w[(int64_t)row * 64 + h] * q_scale[(int64_t)row * 64 + h];
      }
    }
  }

  if (shared && s0 >= 0) {
    // ---- staged path: all rows read sequence s0
    const int32_t* bt_row = block_table + (int64_t)s0 * max_blocks;
    const int kend = min(k1, n_max);
    const int nspans = kend > k0 ? (kend - k0 + kSpan - 1) / kSpan : 0;
    Share reg[2];
    if (nspans > 0) load_share<BS>(reg[0], cache, num_blocks, bt_row, k0, n_max, tid);
    if (nspans > 1) load_share<BS>(reg[1], cache, num_blocks, bt_row, k0 + kSpan, n_max, tid);
    if (nspans > 0) store_share(stage[0], reg[0], tid);
    if (nspans > 2) load_share<BS>(reg[0], cache, num_blocks, bt_row, k0 + 2 * kSpan, n_max, tid);
    __syncthreads();
    for (int i = 0; i < nspans; ++i) {
      // stage[i&1] holds span i; reg[(i+1)&1] holds span i+1; reg[i&1] span i+2
      const uint8_t* st = stage[i & 1];
      const int p_span = k0 + i * kSpan;
      if (active && p_span < n) {
        float val = 0.0f;
        f32x4_t acc[2][4];
        float sg[2];
#pragma unroll
        for (int g = 0; g <= 4; ++g) {
          if (g < 4) {  // LDS reads and MFMAs of group g ...
            const i32x8_t b = read_b(st, g, lane);
            sg[g & 1] = read_scale(st, g, lane);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              acc[g & 1][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  qa[mt], b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
          }
          if (g > 0) {  // ... before the epilogue of group g-1
            const float sc = group_score(acc[(g - 1) & 1], wq, sg[(g - 1) & 1]);
            if ((lane >> 4) == g - 1) val = sc;
          }
        }
        // a block id outside the pool makes the keys it covers NaN
        const int p = p_span + lane;
        const int pb = min(p, n_max - 1);
        const int phys = bt_row[pb / BS];
        if (phys < 0 || phys >= num_blocks) val = __builtin_nanf("");
        if (p >= n) val = -INFINITY;
        if (p < k1 && (p < n || write_pad)) __builtin_nontemporal_store(val, out + p);
      } else if (active && write_pad) {
        const int p = p_span + lane;
        if (p < k1) __builtin_nontemporal_store(-INFINITY, out + p);
      }
      if (i + 1 < nspans) store_share(stage[(i + 1) & 1], reg[(i + 1) & 1], tid);
      if (i + 3 < nspans) load_share<BS>(reg[(i + 1) & 1], cache, num_blocks, bt_row, k0 + (i + 3) * kSpan, n_max, tid);
      __syncthreads();
    }
    if (active && write_pad)  // positions past every key of the workgroup
      for (int p = max(kend, k0) + lane; p < k1; p += 64) out[p] = -INFINITY;
    return;
  }

  // ---- fallback: rows of different sequences, each wave reads its own keys
  if (!active) return;
  const int32_t* bt_row = block_table + (int64_t)seq * max_blocks;
  const int kend = min(k1, n);
  for (int p_span = k0; p_span < kend; p_span += kSpan) {
    float val = 0.0f;
    bool bad = false;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int p0 = p_span + 16 * g;
      if (p0 >= n) continue;  // uniform
      int phys = bt_row[p0 / BS];
      if (phys < 0 || phys >= num_blocks) {
        bad = true;
        phys = 0;
      }
      const uint8_t* blk = cache + (int64_t)phys * (BS * 132);
      const int off = (p0 % BS) + (lane & 15);
      const i32x8_t b = *reinterpret_cast<const i32x8_t*>(blk + off * 128 + 32 * (lane >> 4));
      const float s = reinterpret_cast<const float*>(blk + BS * 128)[off];
      f32x4_t acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            qa[mt], b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      const float sc = group_score(acc, wq, s);
      if ((lane >> 4) == g) val = sc;
    }
    const int p = p_span + lane;
    if (bad && p < n) val = __builtin_nanf("");
    if (p >= n) val = -INFINITY;
    if (p < k1 && (p < n || write_pad)) out[p] = val;
  }
  if (write_pad)
    for (int p = max(kend, k0) + lane; p < k1; p += 64) out[p] = -INFINITY;
}

}  // namespace

hipError_t launch_score_prefill(const uint8_t* q, const float* q_scale, const float* w,
                                const KCache& c, const Rows& r, float* scores, int64_t ld,
                                bool write_pad, hipStream_t s) {
  if (r.rows == 0 || r.max_row_len == 0) return hipSuccess;
  // 8 key chunks, each a whole number of 64-key spans
  const int spans = (r.max_row_len + kSpan - 1) / kSpan;
  const int chunk_keys = (spans + kKeyChunks - 1) / kKeyChunks * kSpan;
  const int tiles = (r.rows + kWavesPf - 1) / kWavesPf;
  const dim3 grid((unsigned)(tiles * kKeyChunks)), block(kThreadsPf);
  if (c.block_size == 64)
    hipLaunchKernelGGL(score_prefill_kernel<64>, grid, block, 0, s, q, q_scale, w, c.base,
                       c.num_blocks, r.block_table, r.max_blocks, r.num_seqs, r.row_seq, r.row_len,
                       r.rows, r.max_row_len, scores, ld, chunk_keys, (int)write_pad);
  else
    hipLaunchKernelGGL(score_prefill_kernel<32>, grid, block, 0, s, q, q_scale, w, c.base,
                       c.num_blocks, r.block_table, r.max_blocks, r.num_seqs, r.row_seq, r.row_len,
                       r.rows, r.max_row_len, scores, ld, chunk_keys, (int)write_pad);
  return hipGetLastError();
}

}  // namespace dsa
