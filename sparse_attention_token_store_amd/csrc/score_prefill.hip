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
//  - Workgroup = 4 waves x 2 query rows = 8 rows; each wave keeps its 2 x 64 heads
//    as 8 A tiles (64 VGPRs) for the whole key loop, so every 16-key B tile loaded
//    feeds 8 MFMAs.  The 4 waves walk the same keys, and the L1 cache serves the
//    repeat reads.
//  - Keys are split into 8 chunks and workgroup w takes chunk w mod 8.  Workgroups
//    are dispatched to the 8 XCDs round robin, so each XCD's L2 only ever holds its
//    eighth of the keys.
//  - Epilogue per 16-key tile: ReLU, weight by w*qs, in-lane head sum over the 16
//    heads a lane holds per row, two cross-lane adds, per-key scale.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kSpan = 64;
constexpr int kRowsPerWave = 2;
constexpr int kRowsPerWg = 4 * kRowsPerWave;
constexpr int kKeyChunks = 8;

struct Raw {
  i32x8_t c[4];  // per 16-key group: this lane's 32 code bytes
  float s[4];    // per group: scale of this lane's key
};

template <int BS>
__device__ __forceinline__ void load_span(Raw& raw, bool& bad, const uint8_t* cache,
                                          int64_t num_blocks, const int32_t* bt_row, int p_span,
                                          int n, int lane) {
  bad = false;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int p0 = p_span + 16 * g;
    if (p0 >= n) continue;  // uniform per wave
    int phys = bt_row[p0 / BS];
    if (phys < 0 || phys >= num_blocks) {
      bad = true;
      phys = 0;
    }
    const int off = (p0 % BS) + (lane & 15);
    const uint8_t* blk = cache + (int64_t)phys * (BS * 132);
    raw.c[g] = *reinterpret_cast<const i32x8_t*>(blk + off * 128 + 32 * (lane >> 4));
    raw.s[g] = reinterpret_cast<const float*>(blk + BS * 128)[off];
  }
}

template <int BS>
__global__ __launch_bounds__(256, 2) void score_prefill_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ cache, int64_t num_blocks, const int32_t* __restrict__ block_table,
    int max_blocks, int num_seqs, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, int rows, int max_row_len, float* __restrict__ scores,
    int64_t ld, int chunk_keys, int write_pad) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk = blockIdx.x % kKeyChunks;
  const int tile = blockIdx.x / kKeyChunks;
  const int r0 = tile * kRowsPerWg + wave * kRowsPerWave;
  const int k0 = chunk * chunk_keys;
  const int k1 = min(k0 + chunk_keys, max_row_len);
  if (r0 >= rows) return;  // a wave past the last row has nothing to read or write

  // this wave's rows (a missing second row is treated as an empty row)
  int rr[kRowsPerWave], nn[kRowsPerWave], sq[kRowsPerWave];
  bool seq_bad[kRowsPerWave];
  int nmax = 0;
#pragma unroll
  for (int t = 0; t < kRowsPerWave; ++t) {
    rr[t] = r0 + t;
    const bool live = rr[t] < rows;
    nn[t] = live ? min(max(row_len[rr[t]], 0), max_row_len) : 0;
    sq[t] = live ? row_seq[rr[t]] : 0;
    seq_bad[t] = live && (sq[t] < 0 || sq[t] >= num_seqs);
    if (!seq_bad[t]) nmax = max(nmax, nn[t]);
  }
  if (k0 >= k1) return;

  // rows whose sequence is out of range score NaN on their visible positions
#pragma unroll
  for (int t = 0; t < kRowsPerWave; ++t)
    if (seq_bad[t])
      for (int p = k0 + lane; p < k1; p += 64) {
        float* o = scores + (int64_t)rr[t] * ld;
        if (p < nn[t]) o[p] = __builtin_nanf("");
        else if (write_pad) o[p] = -INFINITY;
      }

  if (nmax == 0 && !write_pad) return;

  // A operands: row rr[t], head 16*mt + lane%16, code bytes 32*(lane/16) .. +31
  i32x8_t qa[kRowsPerWave][4];
  float wq[kRowsPerWave][4][4];  // w * q_scale of the accumulator rows this lane holds
#pragma unroll
  for (int t = 0; t < kRowsPerWave; ++t) {
    const int r = rr[t] < rows ? rr[t] : r0;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      qa[t][mt] = *reinterpret_cast<const i32x8_t*>(
          q + ((int64_t)r * 64 + 16 * mt + (lane & 15)) * kHeadDim + 32 * (lane >> 4));
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * mt + 4 * (lane >> 4) + v;
        wq[t][mt][v] = w[(int64_t)r * 64 + h] * q_scale[(int64_t)r * 64 + h];
      }
    }
  }

  // One pass over the keys serves both rows when they read the same sequence;
  // rows of different sequences take one pass each.
  const bool live1 = rr[1] < rows && !seq_bad[1];
  const bool shared = !live1 || seq_bad[0] || sq[0] == sq[1];
  const int npass = shared ? 1 : 2;
  for (int pass = 0; pass < npass; ++pass) {
    bool act[kRowsPerWave];
#pragma unroll
    for (int t = 0; t < kRowsPerWave; ++t)
      act[t] = rr[t] < rows && !seq_bad[t] && (shared || t == pass);
    int n = 0, seq = 0;
#pragma unroll
    for (int t = 0; t < kRowsPerWave; ++t)
      if (act[t]) {
        n = max(n, nn[t]);
        seq = sq[t];
      }
    const int32_t* bt_row = block_table + (int64_t)seq * max_blocks;
    const int kend = min(k1, n);

    Raw cur, nxt;
    bool cur_bad = false, nxt_bad = false;
    int p_span = k0;
    if (p_span < kend) load_span<BS>(cur, cur_bad, cache, num_blocks, bt_row, p_span, n, lane);
    for (; p_span < kend; p_span += kSpan) {
      const int p_next = p_span + kSpan;
      if (p_next < kend) load_span<BS>(nxt, nxt_bad, cache, num_blocks, bt_row, p_next, n, lane);
      float val[kRowsPerWave] = {0.0f, 0.0f};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t acc[kRowsPerWave][4];
#pragma unroll
        for (int t = 0; t < kRowsPerWave; ++t) {
          if (!act[t]) continue;  // uniform
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[t][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                qa[t][mt], cur.c[g], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        }
#pragma unroll
        for (int t = 0; t < kRowsPerWave; ++t) {
          if (!act[t]) continue;
          float part = 0.0f;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) part = fmaf(wq[t][mt][v], fmaxf(acc[t][mt][v], 0.0f), part);
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          part *= cur.s[g];
          if ((lane >> 4) == g) val[t] = part + 0.0f;  // a zero score is +0
        }
      }
      const int p = p_span + lane;
#pragma unroll
      for (int t = 0; t < kRowsPerWave; ++t) {
        if (!act[t]) continue;
        float v = p < nn[t] ? val[t] : -INFINITY;
        if (cur_bad && p < nn[t]) v = __builtin_nanf("");
        if (p < k1 && (p < nn[t] || write_pad)) scores[(int64_t)rr[t] * ld + p] = v;
      }
      cur = nxt;
      cur_bad = nxt_bad;
    }
    if (write_pad)  // positions past every key this pass's rows see
#pragma unroll
      for (int t = 0; t < kRowsPerWave; ++t)
        if (act[t])
          for (int p = max(kend, k0) + lane; p < k1; p += 64) scores[(int64_t)rr[t] * ld + p] = -INFINITY;
  }
}

}  // namespace

hipError_t launch_score_prefill(const uint8_t* q, const float* q_scale, const float* w,
                                const KCache& c, const Rows& r, float* scores, int64_t ld,
                                bool write_pad, hipStream_t s) {
  if (r.rows == 0 || r.max_row_len == 0) return hipSuccess;
  // 8 key chunks, each a whole number of 64-key spans
  const int spans = (r.max_row_len + kSpan - 1) / kSpan;
  const int chunk_keys = (spans + kKeyChunks - 1) / kKeyChunks * kSpan;
  const int tiles = (r.rows + kRowsPerWg - 1) / kRowsPerWg;
  const dim3 grid((unsigned)(tiles * kKeyChunks)), block(256);
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
