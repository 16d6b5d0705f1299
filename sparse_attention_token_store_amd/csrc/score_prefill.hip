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
//  - The 8 waves share the keys through LDS: every stage of 256 keys (four 64-token
//    blocks: 32 KB of codes plus 1 KB of scales) is loaded once per workgroup, four
//    16-byte code chunks and one scale per thread, a stage ahead in registers, and
//    copied into a double-buffered LDS stage (75 KB: two workgroups per CU).  Key rows are padded to 144 bytes:
//    16-byte reads of 16 consecutive keys at the same offset then fall on 16
//    distinct bank groups (9r mod 16 is a permutation), so the B-operand reads,
//    lane = (key, 32-byte quarter), do not conflict.  A key whose block id lies
//    outside the pool is staged with a NaN scale, so its score is NaN without any
//    check in the scoring loop.  About 120 VGPRs per wave: 4 waves per SIMD.
//  - The stage barrier orders LDS only (the global prefetch stays in flight across
//    it), every thread issues the same loads each stage (positions past the last
//    key clamped to it) so the compiler's load-counter waits stay exact, and the
//    block-table entries are fetched a stage before the keys they locate.
//  - The matrix core and the VALU overlap across the 4 waves of a SIMD (within one
//    wave they largely take turns), so each 16-key group is scored in place.
//  - Keys are split into 8 chunks and workgroup w takes chunk w mod 8.  Workgroups
//    are dispatched to the 8 XCDs round robin, so each XCD's L2 only ever holds its
//    eighth of the keys.
//  - Epilogue per 16-key tile: ReLU, weight by w*qs, in-lane head sum over the 16
//    heads a lane holds; then per 64 keys one reduce-scatter over the four lane-rows
//    (3 permlane swaps) and one per-key scale, so lane l holds key l of the span.
//  - A workgroup whose rows read different sequences falls back to per-wave direct
//    loads (correct, slower; chunked prefill never takes it).
//  - MXFP4 keys (e2m1 codes + an e8m0 scale per 32 dims) take the same path with the
//    MFMA's B format set to fp4: a lane's 32 contiguous dims are one scale block, so
//    its key's e8m0 byte for that block is the lane's B scale operand and the
//    per-key factor of the epilogue is 1 (NaN for a key of a bad block id).  Staged
//    key rows are 64 bytes padded to 80 (80/16 odd: still 16 distinct bank groups).
#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kSpan = 64;                   // keys per score store (one per lane)
constexpr int kWavesPf = 8;                 // one query row per wave
constexpr int kThreadsPf = 64 * kWavesPf;
constexpr int kKeyChunks = 8;
constexpr int kStageKeys = 256;                         // keys per LDS stage
constexpr int kStageGroups = kStageKeys / 16;
constexpr int kRowPitch = 144;                          // padded LDS key row (fp8)
constexpr int kScaleOff = kStageKeys * kRowPitch;       // scales after the key rows
constexpr int kStage = kScaleOff + kStageKeys * 4;      // 37,888 bytes per stage
constexpr int kRowPitch4 = 80;                          // padded LDS key row (MXFP4)
constexpr int kScaleOff4 = kStageKeys * kRowPitch4;     // e8m0 words after the key rows
constexpr uint32_t kBadKey = 0xFFFFFFFFu;               // staged e8m0 word of a bad block

// One thread's share of a stage: code chunk tid & 7 of keys 64j + (tid >> 3), j < 4,
// and the scale of key tid % 256 (threads 0..255 stage it).  Every thread issues the
// same loads every stage, with positions past the last key clamped to it: with no
// skipped loads the compiler's load-counter waits stay exact.  (Keys past a row's
// end are overwritten with -inf, so what the clamped loads bring is never used.)
// Named fields, not arrays: an aggregate array here ends up in scratch memory.
struct Share {
  uint4 c0, c1, c2, c3;
  uint32_t scale;
};

// Block-table entries behind one thread's share of the stage at p0, fetched a stage
// before the share itself so the key loads never wait on a block-table load.
struct ShareBlocks {
  int b0, b1, b2, b3, scale;
};

// (Positions are non-negative: unsigned arithmetic makes / BS and % BS shifts and masks.)
template <int BS, bool kFp4>
__device__ __forceinline__ ShareBlocks share_blocks(const int32_t* bt_row, int p0, int n_max, int tid) {
  const uint32_t last = (uint32_t)n_max - 1u;
  const uint32_t ks = (uint32_t)p0 + ((uint32_t)tid & 255u);
  if constexpr (kFp4) {  // code chunk tid & 3 of keys tid >> 2 and 128 + (tid >> 2)
    const uint32_t k = (uint32_t)p0 + ((uint32_t)tid >> 2);
    return ShareBlocks{bt_row[min(k, last) / BS], bt_row[min(k + 128u, last) / BS], 0, 0,
                       bt_row[min(ks, last) / BS]};
  } else {
    const uint32_t k = (uint32_t)p0 + ((uint32_t)tid >> 3);
    return ShareBlocks{bt_row[min(k, last) / BS], bt_row[min(k + 64u, last) / BS], bt_row[min(k + 128u, last) / BS],
                       bt_row[min(k + 192u, last) / BS], bt_row[min(ks, last) / BS]};
  }
}

template <int BS>
__device__ __forceinline__ uint4 load_code(const uint8_t* cache, int64_t num_blocks, int entry, uint32_t pos, int tid) {
  const uint32_t phys = (entry < 0 || entry >= num_blocks) ? 0u : (uint32_t)entry;
  return *reinterpret_cast<const uint4*>(cache + (uint64_t)phys * (BS * 132) +
                                         ((pos % BS) * 128u + ((uint32_t)tid & 7u) * 16u));
}

// MXFP4: code chunk tid & 3 (16 bytes) of the key at pos, and a key's e8m0 word
template <int BS>
__device__ __forceinline__ uint4 load_code4(const uint8_t* cache, int64_t num_blocks, int entry, uint32_t pos, int tid) {
  const uint32_t phys = (entry < 0 || entry >= num_blocks) ? 0u : (uint32_t)entry;
  return *reinterpret_cast<const uint4*>(cache + (uint64_t)phys * (BS * 68) +
                                         ((pos % BS) * 64u + ((uint32_t)tid & 3u) * 16u));
}

template <int BS, bool kFp4>
__device__ __forceinline__ Share load_share(const uint8_t* cache, int64_t num_blocks, const ShareBlocks& e,
                                            int p0, int n_max, int tid) {
  const uint32_t last = (uint32_t)n_max - 1u;
  Share sh;
  if constexpr (kFp4) {
    const uint32_t k = (uint32_t)p0 + ((uint32_t)tid >> 2);
    sh.c0 = load_code4<BS>(cache, num_blocks, e.b0, min(k, last), tid);
    sh.c1 = load_code4<BS>(cache, num_blocks, e.b1, min(k + 128u, last), tid);
    sh.c2 = sh.c3 = make_uint4(0, 0, 0, 0);
    const uint32_t ps = min((uint32_t)p0 + ((uint32_t)tid & 255u), last);
    const bool bad = e.scale < 0 || e.scale >= num_blocks;
    const uint32_t v = *reinterpret_cast<const uint32_t*>(cache + (uint64_t)(bad ? 0u : (uint32_t)e.scale) * (BS * 68) +
                                                          (BS * 64u + (ps % BS) * 4u));
    sh.scale = bad ? kBadKey : v;
    return sh;
  }
  const uint32_t k = (uint32_t)p0 + ((uint32_t)tid >> 3);
  sh.c0 = load_code<BS>(cache, num_blocks, e.b0, min(k, last), tid);
  sh.c1 = load_code<BS>(cache, num_blocks, e.b1, min(k + 64u, last), tid);
  sh.c2 = load_code<BS>(cache, num_blocks, e.b2, min(k + 128u, last), tid);
  sh.c3 = load_code<BS>(cache, num_blocks, e.b3, min(k + 192u, last), tid);
  // a block id outside the pool stages a NaN scale: its keys score NaN
  const uint32_t ps = min((uint32_t)p0 + ((uint32_t)tid & 255u), last);
  const bool bad = e.scale < 0 || e.scale >= num_blocks;
  const uint32_t v = *reinterpret_cast<const uint32_t*>(cache + (uint64_t)(bad ? 0u : (uint32_t)e.scale) * (BS * 132) +
                                                        (BS * 128u + (ps % BS) * 4u));
  sh.scale = bad ? 0x7FC00000u : v;
  return sh;
}

// Block size 64, fp8 keys, a stage wholly below the workgroup's longest row: the
// stage's 256 keys fill four whole blocks, each thread's four code chunks come one
// from each (chunk tid & 7 of key tid >> 3 of the block) and the scales of wave w
// from block w & 3, so the four block ids are uniform (scalar loads) and a code
// address is a uniform block base plus a per-thread offset that is the same in
// every stage.
__device__ __forceinline__ Share load_share_whole64(const uint8_t* cache, int64_t num_blocks,
                                                    const int32_t* bt_row, int p0, int tid, int wave) {
  constexpr uint32_t kBlockBytes = 64 * 132;
  const uint32_t off = (uint32_t)(tid >> 3) * 128u + (uint32_t)(tid & 7) * 16u;
  const uint8_t* base[4];
  bool bad[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = bt_row[(p0 >> 6) + j];
    bad[j] = e < 0 || (int64_t)e >= num_blocks;
    base[j] = cache + (uint64_t)(bad[j] ? 0u : (uint32_t)e) * kBlockBytes;
  }
  Share sh;
  sh.c0 = *reinterpret_cast<const uint4*>(base[0] + off);
  sh.c1 = *reinterpret_cast<const uint4*>(base[1] + off);
  sh.c2 = *reinterpret_cast<const uint4*>(base[2] + off);
  sh.c3 = *reinterpret_cast<const uint4*>(base[3] + off);
  const int j = wave & 3;
  const uint8_t* sb = j == 0 ? base[0] : j == 1 ? base[1] : j == 2 ? base[2] : base[3];
  const bool sbad = j == 0 ? bad[0] : j == 1 ? bad[1] : j == 2 ? bad[2] : bad[3];
  const uint32_t v = *reinterpret_cast<const uint32_t*>(sb + 64u * 128u + (uint32_t)(tid & 63) * 4u);
  sh.scale = sbad ? 0x7FC00000u : v;  // a block id outside the pool: NaN scores
  return sh;
}

template <bool kFp4>
__device__ __forceinline__ void store_share(uint8_t* stage, const Share& sh, int tid) {
  if constexpr (kFp4) {
    uint8_t* p = stage + (tid >> 2) * kRowPitch4 + (tid & 3) * 16;
    *reinterpret_cast<uint4*>(p) = sh.c0;
    *reinterpret_cast<uint4*>(p + 128 * kRowPitch4) = sh.c1;
    if (tid < kStageKeys) reinterpret_cast<uint32_t*>(stage + kScaleOff4)[tid] = sh.scale;
    return;
  }
  uint8_t* p = stage + (tid >> 3) * kRowPitch + (tid & 7) * 16;
  *reinterpret_cast<uint4*>(p) = sh.c0;
  *reinterpret_cast<uint4*>(p + 64 * kRowPitch) = sh.c1;
  *reinterpret_cast<uint4*>(p + 128 * kRowPitch) = sh.c2;
  *reinterpret_cast<uint4*>(p + 192 * kRowPitch) = sh.c3;
  if (tid < kStageKeys) reinterpret_cast<uint32_t*>(stage + kScaleOff)[tid] = sh.scale;
}

// B operand of group g for this lane: key 16g + lane%16, code bytes 32*(lane/16) .. +31
__device__ __forceinline__ i32x8_t read_b(const uint8_t* stage, int g, int lane) {
  const uint8_t* p = stage + (16 * g + (lane & 15)) * kRowPitch + 32 * (lane >> 4);
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}
// MXFP4: key 16g + lane%16, code bytes 16*(lane/16) .. +15 (32 e2m1, one scale block)
__device__ __forceinline__ i32x8_t read_b4(const uint8_t* stage, int g, int lane) {
  const uint4 c = *reinterpret_cast<const uint4*>(stage + (16 * g + (lane & 15)) * kRowPitch4 + 16 * (lane >> 4));
  return i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
}
// the e8m0 byte of this lane's scale block (B scale operand of the MFMA)
__device__ __forceinline__ int scale_b4(uint32_t word, int lane) { return (int)((word >> (8 * (lane >> 4))) & 0xFFu); }
// epilogue factor of a key from its staged e8m0 word: 1, or NaN for a bad block id
__device__ __forceinline__ float key_factor4(uint32_t word) {
  return word == kBadKey ? __builtin_nanf("") : 1.0f;
}

// In-lane part of the epilogue of one 16-key group: the ReLU-weighted sum over the
// 16 heads this lane holds, for key lane%16 of the group.
__device__ __forceinline__ float group_part(const f32x4_t (&acc)[4], const float (&wq)[4][4]) {
  float part = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) part = fmaf(wq[mt][v], relu(acc[mt][v]), part);
  return part;
}

// Epilogue of one 16-key group for the per-wave direct path: the row's score for key
// 16g + lane%16 (in every 16-lane row of the wave).
__device__ __forceinline__ float group_score(const f32x4_t (&acc)[4], const float (&wq)[4][4], float s) {
  return rows4_sum(group_part(acc, wq)) * s + 0.0f;  // +0.0f: a zero score is +0
}

template <int BS, bool kFp4>
__global__ __launch_bounds__(kThreadsPf, 4) void score_prefill_kernel(
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

  // A operands of this row: head 16*mt + lane%16, code bytes 32*(lane/16) .. +31.
  // With fp4 B operands the MFMA pairs nibble j of B lane group g with A contraction
  // slot k = 16*(g>>1) + 64*(g&1) + 32*(j>>4) + (j&15), where slot k is byte k%32 of
  // A lane group k/32 (measured on the hardware for all 64 x 32 nibbles), and a B
  // lane's scale byte scales its own 32 nibbles.  B lane group g holds the 32-dim
  // scale block g (dims 32g + j), so A lane group a holds dims 16a .. 16a+15 in bytes
  // 0..15 and 64+16a .. 64+16a+15 in bytes 16..31.
  i32x8_t qa[4];
  float wq[4][4];  // w * q_scale of the accumulator rows this lane holds
  if (active) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint8_t* qh = q + ((int64_t)row * 64 + 16 * mt + (lane & 15)) * kHeadDim;
      if constexpr (kFp4) {
        const uint4 lo = *reinterpret_cast<const uint4*>(qh + 16 * (lane >> 4));
        const uint4 hi = *reinterpret_cast<const uint4*>(qh + 64 + 16 * (lane >> 4));
        qa[mt] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      } else {
        qa[mt] = *reinterpret_cast<const i32x8_t*>(qh + 32 * (lane >> 4));
      }
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
    const int nst = kend > k0 ? (kend - k0 + kStageKeys - 1) / kStageKeys : 0;
    if (nst == 0) {  // no key of the chunk is visible to any row
      if (active && write_pad)
        for (int p = k0 + lane; p < k1; p += 64) out[p] = -INFINITY;
      return;
    }
    // (uniform copies: the scalar path below needs the compiler to know it)
    const int n_max_u = __builtin_amdgcn_readfirstlane(n_max);
    const int32_t* bt_row_u = block_table + (int64_t)__builtin_amdgcn_readfirstlane(s0) * max_blocks;
    auto whole = [&](int i) {  // (uniform) stage i takes the scalar path
      if constexpr (BS == 64 && !kFp4) return k0 + i * kStageKeys + kStageKeys <= n_max_u;
      return false;
    };
    auto blocks = [&](int i) {
      if (whole(i)) return ShareBlocks{0, 0, 0, 0, 0};  // (not used)
      return share_blocks<BS, kFp4>(bt_row, k0 + i * kStageKeys, n_max, tid);
    };
    auto share = [&](const ShareBlocks& e, int i) {
      if (whole(i)) return load_share_whole64(cache, num_blocks, bt_row_u, k0 + i * kStageKeys, tid, wave);
      return load_share<BS, kFp4>(cache, num_blocks, e, k0 + i * kStageKeys, n_max, tid);
    };
    // Scores stage i from the staged copy st: groups of 16 keys, one 64-key store
    // per 4 groups (reads the row's operands only).
    auto score_stage = [&](int i, const uint8_t* st) {
      const int p0 = k0 + i * kStageKeys;
      if (!active) return;
      if (p0 >= n) {  // none of these keys is visible to this row
        if (write_pad)
          for (int p = p0 + lane; p < min(p0 + kStageKeys, k1); p += 64) __builtin_nontemporal_store(-INFINITY, out + p);
        return;
      }
      float part[4];
#pragma unroll
      for (int g = 0; g < kStageGroups; ++g) {
        // A group's four MFMAs issue together and its epilogue follows them: the
        // scheduling barriers keep the compiler from interleaving one group's
        // epilogue with the next group's MFMAs (1165-1189 -> 1135-1137 us on the
        // 4096 x 36,864 prefill; the four waves of a SIMD overlap the two instead).
        f32x4_t acc[4];
        if constexpr (kFp4) {
          const i32x8_t b = read_b4(st, g, lane);
          const int sb = scale_b4(reinterpret_cast<const uint32_t*>(st + kScaleOff4)[16 * g + (lane & 15)], lane);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)  // A: fp8 e4m3 at scale 2^0; B: fp4 e2m1 at its block scale
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                qa[mt], b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sb);
        } else {
          const i32x8_t b = read_b(st, g, lane);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                qa[mt], b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        }
        __builtin_amdgcn_sched_barrier(0);
        part[g & 3] = group_part(acc, wq);
        if ((g & 3) == 3) {  // 64 keys done: lane l gets key l of the span, one store
          const int sp = g >> 2;
          float sk;
          if constexpr (kFp4)
            sk = key_factor4(reinterpret_cast<const uint32_t*>(st + kScaleOff4)[64 * sp + lane]);
          else
            sk = reinterpret_cast<const float*>(st + kScaleOff)[64 * sp + lane];
          const float v0 = rows4_reduce_scatter(part[0], part[1], part[2], part[3]) * sk + 0.0f;
          const int p = p0 + 64 * sp + lane;
          const float v = p >= n ? -INFINITY : v0;  // (+0.0f above: a zero score is +0)
          if (p < k1 && (p < n || write_pad)) __builtin_nontemporal_store(v, out + p);
        }
      }
    };
    // Iteration i copies stage i+1 (loaded during iteration i-1) from registers into
    // the free LDS buffer, fetches stage i+3's block entries and issues stage i+2's
    // loads into the same registers, then scores stage i.
    Share r = share(blocks(0), 0);
    store_share<kFp4>(stage[0], r, tid);
    r = share(blocks(1), 1);
    ShareBlocks next = blocks(2);  // block entries of stage i+2 at the top of iteration i
    lds_barrier();
    for (int i = 0; i < nst; ++i) {
      if (i + 1 < nst) store_share<kFp4>(stage[(i + 1) & 1], r, tid);
      {
        const ShareBlocks e = next;
        next = blocks(i + 3);
        r = share(e, i + 2);
      }
      score_stage(i, stage[i & 1]);
      lds_barrier();  // (the prefetched stage stays in flight)
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
      const int off = (p0 % BS) + (lane & 15);
      f32x4_t acc[4];
      float s;
      if constexpr (kFp4) {
        const uint8_t* blk = cache + (int64_t)phys * (BS * 68);
        const uint4 c = *reinterpret_cast<const uint4*>(blk + off * 64 + 16 * (lane >> 4));
        const i32x8_t b = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        const int sb = scale_b4(*reinterpret_cast<const uint32_t*>(blk + BS * 64 + off * 4), lane);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              qa[mt], b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sb);
        s = 1.0f;
      } else {
        const uint8_t* blk = cache + (int64_t)phys * (BS * 132);
        const i32x8_t b = *reinterpret_cast<const i32x8_t*>(blk + off * 128 + 32 * (lane >> 4));
        s = reinterpret_cast<const float*>(blk + BS * 128)[off];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              qa[mt], b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      }
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
#define DSA_PF_LAUNCH(BSV, FP4)                                                                     \
  hipLaunchKernelGGL((score_prefill_kernel<BSV, FP4>), grid, block, 0, s, q, q_scale, w, c.base,     \
                     c.num_blocks, r.block_table, r.max_blocks, r.num_seqs, r.row_seq, r.row_len, \
                     r.rows, r.max_row_len, scores, ld, chunk_keys, (int)write_pad)
  const bool fp4 = c.dtype == 3;
  if (c.block_size == 64) {
    if (fp4) DSA_PF_LAUNCH(64, true);
    else DSA_PF_LAUNCH(64, false);
  } else {
    if (fp4) DSA_PF_LAUNCH(32, true);
    else DSA_PF_LAUNCH(32, false);
  }
#undef DSA_PF_LAUNCH
  return hipGetLastError();
}

}  // namespace dsa
