// Causal top-k of fp32 score rows: the k largest scores among positions
// p < row_len, ties to the lower position, output in ascending position order and
// padded with -1 (ROCm/ATOM issue 1507, "Summary": index_topk 512/1024; "How it was
// isolated": the per-row top-k must agree exactly with torch.topk).
//
// Exact selection on order-preserving 32-bit keys, one 1024-thread workgroup per
// chunk of up to 36,864 elements held in registers.  Thread t holds, for each
// group g < R/4, the four consecutive elements g*4096 + 4t .. +3 (one 16-byte load),
// so every position-ordered scan runs once per group of four, on packed counts.
//  1. Lower bound.  Every thread splits its keys into four sets (element e of each
//     of its groups) and takes each set's maximum: 4096 distinct elements of the
//     chunk, so any value t_lo with at least k of them at or above it has
//     tau >= t_lo, tau being the k-th largest key.  t_lo is the lower edge of the
//     histogram bin holding the k-th largest of them (k <= 4096).
//     Keys below t_lo (typically 95-97% of a row) take no further part.
//  2. The live keys (>= t_lo) are compacted, in position order, into an LDS list
//     with their positions.  (If they do not fit, e.g. long runs of equal scores,
//     the same steps run over the registers instead.)
//  3. Radix search for tau: an LDS histogram of up to 2048 bins over the 11 bits
//     just below the common prefix of t_lo and the row maximum, where the live keys
//     actually differ; one wavefront scans the bins from the top.  A boundary bin of
//     at most 128 keys is settled by ranking its keys against each other, otherwise
//     11 more bits at a time.
//  4. Every key above tau is kept plus the first `rem` keys equal to it: with
//     position-ordered counts G (greater) and E (equal) of the keys before a key,
//     its output slot is G + min(E, rem).
//  5. Optionally (a slot map is given) the last level translates its selections to
//     physical cache slots in one pass after every emit.
// Rows longer than one chunk are reduced level by level: each chunk keeps its own
// top-k (exact: an element of the row's top-k under the order (score desc,
// position asc) is also in its chunk's top-k), the survivors stay in position
// order, and the next level selects among them.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLevel0Chunk = 16384;    // first reducing level of long rows (R = 16), or twice that
constexpr int kLevelNChunk = 32768;    // largest chunk of the later reducing levels (R = 32)
constexpr int kMaxR = 36;
constexpr int kMaxSingle = kMaxR * kThreads;   // 36,864: one chunk
constexpr uint32_t kMinKey = 1u << 21;  // floor of the lower bound (below every real key)
constexpr int kListMax = 8192;          // live keys held in the LDS list
constexpr int kRankMax = 128;           // boundary bins this small are settled by ranking

// Score -> unsigned key with the same order (larger score, larger key), in the order
// torch.topk ranks values.  A non-negative score gets the top bit set; a negative one
// becomes its two's complement, which reverses the order of the negative scores and
// puts -0 on the key of +0 (0x80000000).  The smallest key, that of -inf, is 0x00800000.
// NaNs are left to nan_key: here a NaN of positive sign lands above the key of +inf
// and one of negative sign below the key of -inf.
__device__ __forceinline__ uint32_t order_key_raw(uint32_t u) {
  return (int32_t)u < 0 ? 0u - u : (u | 0x80000000u);
}
// Every NaN, of either sign and any payload, takes the largest key, above +inf (NaNs
// tie among themselves); other keys, and the sentinel 0, pass unchanged.
__device__ __forceinline__ uint32_t nan_key(uint32_t key) {
  return (key > 0xFF800000u || key - 1u < 0x007FFFFFu) ? 0xFFFFFFFFu : key;
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : 0u - k);
}

// number of candidates a row keeps after one level with chunk size C
__device__ __host__ __forceinline__ int64_t after_level(int64_t n, int64_t C, int k) {
  const int64_t full = n / C, rest = n - full * C;
  return full * (k < C ? k : C) + (rest < k ? rest : k);
}

struct Lists {  // candidate lists of one level: keys and positions, [rows][cap], cap % 4 == 0
  uint32_t* keys;
  int32_t* idx;
  int64_t cap;
};

// Levels a row can need: the first level halves a row at worst (k = 8192 keeps 8192
// of every 16,384), every later one keeps at most 1 in 4 (k of >= 4k), so a row of
// INT32_MAX elements reaches one 36,864-element chunk after 9 reducing levels (10
// with the last); 12 leaves room.
constexpr int kMaxLevels = 12;

struct LevelChunks {  // chunk size of every level, passed by value
  int64_t c[kMaxLevels];
};

// Inclusive scan over the 64 lanes of a wavefront with the gfx9 DPP row shifts:
// shifts by 1, 2, 4, 8 within each row of 16 lanes, then row_bcast:15 carries row
// 0's and row 2's last lane into rows 1 and 3, and row_bcast:31 carries lane 31
// into rows 2 and 3.  Lanes without a source take the identity.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t x, uint32_t id, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
// inclusive prefix sum over the lanes (unsigned: packed counts)
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  return wave_scan_dpp(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = wave_scan_dpp(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = wave_scan_dpp(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Run by one wavefront: find the bin (of nbins = 64 * PER, or fewer when PER = 1)
// that holds the rem-th largest counted key, scanning from the top bin down.
// Lane l owns the PER contiguous bins [nbins - (l+1)*PER, nbins - l*PER).  First
// every lane sums its bins (reading its 16-byte pieces in a lane-rotated order, so
// that lanes PER words apart do not all hit one LDS bank) and a prefix sum over the
// lanes finds the lane whose bins hold the rem-th key; then PER lanes take one bin
// each of that lane's range, top bin first, and a second prefix sum finds the bin.
// Writes info = {bin, count above the bin, count in it}; nothing when fewer than
// rem keys were counted.
template <int PER>
__device__ __forceinline__ void find_bin_t(const int* hist, int nbins, int rem, int* info) {
  const int lane = lane_id();
  const int lo = nbins - (lane + 1) * PER;
  int cnt = 0;
  if (lo >= 0) {
    if constexpr (PER >= 4) {
#pragma unroll
      for (int q = 0; q < PER / 4; ++q) {
        const int qq = (q + lane) & (PER / 4 - 1);
        const int4 v = reinterpret_cast<const int4*>(hist + lo)[qq];
        cnt += v.x + v.y + v.z + v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < PER; ++q) cnt += hist[lo + q];
    }
  }
  const int x = (int)wave_incl_scan((uint32_t)cnt);  // this lane's bins and all above
  const uint64_t hit = __ballot(x >= rem);           // (x does not decrease with the lane)
  if (hit == 0) return;
  const int L = __builtin_ctzll(hit);
  const int above = __builtin_amdgcn_readlane(x - cnt, L);
  const int top = nbins - L * PER - 1;  // lane L's top bin
  const int h = lane < PER ? hist[top - lane] : 0;
  const int y = (int)wave_incl_scan((uint32_t)h) + above;
  const int J = __builtin_ctzll(__ballot(lane < PER && y >= rem));
  if (lane == J) {
    info[0] = top - J;
    info[1] = y - h;
    info[2] = h;
  }
}

__device__ __forceinline__ void find_bin(const int* hist, int nbins, int rem, int* info) {
  switch (nbins >> 6) {
    case 32: find_bin_t<32>(hist, nbins, rem, info); break;
    case 16: find_bin_t<16>(hist, nbins, rem, info); break;
    case 8: find_bin_t<8>(hist, nbins, rem, info); break;
    case 4: find_bin_t<4>(hist, nbins, rem, info); break;
    case 2: find_bin_t<2>(hist, nbins, rem, info); break;
    default: find_bin_t<1>(hist, nbins, rem, info); break;
  }
}

// One wavefront turns the per-(group, wave) packed counts tab[0..E) into exclusive
// offsets in position order (group-major, then wave) and stores the sum in *total.
__device__ __forceinline__ void scan_table(uint32_t* tab, int E, uint32_t* total) {
  const int lane = lane_id();
  const int per = (E + 63) / 64, e0 = lane * per;
  uint32_t sum = 0;
  for (int q = 0; q < per; ++q)
    if (e0 + q < E) sum += tab[e0 + q];
  const uint32_t incl = wave_incl_scan(sum);
  uint32_t run = incl - sum;
  for (int q = 0; q < per; ++q)
    if (e0 + q < E) {
      const uint32_t v = tab[e0 + q];
      tab[e0 + q] = run;
      run += v;
    }
  if (lane == 63) *total = incl;
}

// Every wavefront reads the per-(group, wave) counts tab[0..G*kWaves) itself and
// takes the exclusive offsets of its own entries in position order (group-major,
// then wave) and the total: no single-wave pass and no second barrier.  Entry
// g*kWaves + w sits in lane 16*(g%4) + w of scan g/4 (kWaves = 16).
template <int G>
__device__ __forceinline__ void table_offsets(const uint32_t* tab, int wave, uint32_t (&off)[G], uint32_t& total) {
  static_assert(kWaves == 16, "four groups per 64-entry scan");
  constexpr int E = G * kWaves, J = (E + 63) / 64;
  const int lane = lane_id();
  uint32_t ex[J];
  uint32_t base = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = 64 * j + lane;
    const uint32_t x = i < E ? tab[i] : 0u;
    const uint32_t inc = wave_incl_scan(x);
    ex[j] = inc - x + base;
    base += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  }
  total = base;
#pragma unroll
  for (int g = 0; g < G; ++g) off[g] = (uint32_t)__builtin_amdgcn_readlane((int)ex[g >> 2], 16 * (g & 3) + wave);
}

// Physical cache slot of key position t of row r (the paged layout of the store:
// logical block t / bs at offset t % bs, the block table naming the physical block),
// or -1 when t is not a visible position of the row or a sequence or block id lies
// outside its table.
__device__ __forceinline__ int64_t physical_slot(const SlotMap& m, int64_t r, int32_t t) {
  const int seq = m.row_seq[r];
  const int len = min(max(m.row_len[r], 0), m.max_row_len);
  if ((unsigned)seq >= (unsigned)m.num_seqs || t < 0 || t >= len) return -1;
  const int lb = t / m.block_size;
  if (lb >= m.max_blocks) return -1;
  const int32_t b = m.block_table[(int64_t)seq * m.max_blocks + lb];
  if (b < 0 || (int64_t)b >= m.num_blocks) return -1;
  return (int64_t)b * m.block_size + (t - lb * m.block_size);
}

// kFirst: source is the score matrix; else a candidate list.  kLast: write the
// final out_idx / out_scores (and the slots of map); else the next candidate list.  kVec: 16-byte loads of
// the source are aligned (score rows with ld % 4 == 0; lists always).
template <int R, bool kFirst, bool kLast, bool kVec>
__global__ __launch_bounds__(kThreads) void topk_level_kernel(
    const float* __restrict__ scores, int64_t ld, Lists src, Lists dst,
    const int32_t* __restrict__ row_len, int max_row_len, int k, int nlevel, LevelChunks chunks,
    int32_t* __restrict__ out_idx, float* __restrict__ out_scores, SlotMap map) {
  static_assert(R % 4 == 0, "slots come in groups of four");
  constexpr int G = R / 4;             // groups of four per thread
  constexpr int C = R * kThreads;      // chunk length
  constexpr int E = G * kWaves;        // (group, wave) entries of the ordered scans
  __shared__ __attribute__((aligned(16))) int hist[2048];
  __shared__ uint32_t lkey[kListMax];
  __shared__ int32_t lpos[kListMax];
  __shared__ uint32_t tab[E];
  __shared__ uint32_t wtot[kWaves];
  __shared__ uint32_t red_max[kWaves], red_min[kWaves];
  __shared__ int info[3];
  __shared__ uint32_t total;
  __shared__ int ncand;
  __shared__ uint32_t tau_key;
  __shared__ int tau_gt;

  const int r = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;

  // elements of this row at this level
  int64_t n = min(max(row_len[r], 0), max_row_len);
  for (int l = 0; l < nlevel; ++l) n = after_level(n, chunks.c[l], k);
  const int64_t base = (int64_t)c * C;
  const int nc = (int)max((int64_t)0, min((int64_t)C, n - base));

  if constexpr (kLast) {  // one chunk per row: slots nc..k-1 are padding
    for (int p = nc + tid; p < k; p += kThreads) {
      out_idx[(int64_t)r * k + p] = -1;
      if (out_scores) out_scores[(int64_t)r * k + p] = -INFINITY;
      if (map.slots) map.slots[(int64_t)r * map.ld + p] = -1;
    }
  }
  if (nc <= 0) return;

  // element 4*g + e of this thread sits at chunk offset li(g, e)
  auto li_of = [&](int g, int e) { return g * 4 * kThreads + 4 * tid + e; };

  // Slots past the chunk's end hold the sentinel key 0; a real key is at least
  // 0x00800000 (-inf) and the lower bound is never below kMinKey = 2^21, so the
  // sentinel is never counted or selected.
  // Every load is issued before the first is consumed: the loads take no branch
  // (a group past the chunk's end reads the chunk's first elements instead, and
  // its values are then masked), so their latencies overlap.
  uint32_t key[R];
  {
    uint32_t raw[R];
    if constexpr (!kFirst || kVec) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // The longest chunks (R = 36, one chunk per prefill row): l0 itself when
        // l0 < nc (a multiple of 4 at most nc - 1), else the chunk's last whole four,
        // with no compare mask kept alive (fewer spilled SGPRs: prefill 220 -> 213 us).
        // Shorter chunks keep reading the first four for groups past the end, which
        // measured faster there (decode_b32 rows 9.54 against 9.76 us, the 32,768-key
        // levels of 1M-key rows 25.5 against 26.1 us).
        const int l0 = li_of(g, 0);
        const int at = R >= kMaxR ? min(l0, (nc - 1) & ~3) : (l0 < nc ? l0 : 0);
        uint4 v;
        if constexpr (kFirst)
          v = *reinterpret_cast<const uint4*>(scores + (int64_t)r * ld + base + at);
        else
          v = *reinterpret_cast<const uint4*>(src.keys + (int64_t)r * src.cap + base + at);
        raw[4 * g] = v.x;
        raw[4 * g + 1] = v.y;
        raw[4 * g + 2] = v.z;
        raw[4 * g + 3] = v.w;
      }
    } else {  // rows not 16-byte aligned: element loads, clamped into the chunk
      const float* p = scores + (int64_t)r * ld + base;
#pragma unroll
      for (int j = 0; j < R; ++j) raw[j] = __float_as_uint(p[min(li_of(j >> 2, j & 3), nc - 1)]);
    }
    uint64_t nan_lanes = 0;  // lanes of this wave that loaded a NaN score
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if constexpr (kFirst) {
        nan_lanes |= __ballot(__builtin_isnan(__uint_as_float(raw[j])));
        key[j] = order_key_raw(raw[j]);
      } else {
        key[j] = raw[j];
      }
    }
    if (nan_lanes != 0) {  // (uniform; rare)
#pragma unroll
      for (int j = 0; j < R; ++j) key[j] = nan_key(key[j]);
    }
    // only the groups that reach past the chunk's end hold slots to mask (uniform test)
#pragma unroll
    for (int g = 0; g < G; ++g)
      if ((g + 1) * 4 * kThreads > nc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * g + e] = li_of(g, e) < nc ? key[4 * g + e] : 0u;
      }
  }

  auto emit = [&](int pos, int li, uint32_t kv) {
    // (never taken: exactly k keys are selected, each from this chunk)
    if ((unsigned)pos >= (unsigned)k || (unsigned)li >= (unsigned)nc) return;
    int32_t idx;
    if constexpr (kFirst)
      idx = (int32_t)(base + li);
    else
      idx = src.idx[(int64_t)r * src.cap + base + li];
    if constexpr (kLast) {
      out_idx[(int64_t)r * k + pos] = idx;
      if (out_scores) out_scores[(int64_t)r * k + pos] = key_to_float(kv);
    } else {
      const int64_t o = (int64_t)r * dst.cap + (int64_t)c * k + pos;
      dst.keys[o] = kv;
      dst.idx[o] = idx;
    }
  };

  // 5. (last level, with a slot map) the physical slot of every selection: one pass
  // over this row's out_idx after every emit, read back from L2 once the barrier has
  // made the workgroup's writes visible, so each selection costs one table gather.
  auto finish_slots = [&]() {
    if constexpr (kLast) {
      if (map.slots) {
        __syncthreads();
        const int m = min(nc, k);
        for (int p = tid; p < m; p += kThreads)
          map.slots[(int64_t)r * map.ld + p] = physical_slot(map, r, out_idx[(int64_t)r * k + p]);
      }
    }
  };

  if (nc <= k) {  // everything survives, in order
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int li = li_of(j >> 2, j & 3);
      if (li < nc) emit(li, li, key[j]);
    }
    finish_slots();
    return;
  }

  // ---- 1. row maximum and the lower bound t_lo: the k-th largest of the 4096
  // values formed by every thread's four set maxima (set e holds the thread's keys
  // 4g + e over its groups g), each a distinct element of the chunk, so at least k
  // keys lie at or above it; located to an 11-bit histogram bin and rounded down to
  // that bin's lower edge
  for (int b = tid; b < 2048; b += kThreads) hist[b] = 0;
  uint32_t sm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm[e] = max(sm[e], key[4 * g + e]);
  const uint32_t m1 = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
  {
    // the smallest maximum over threads that hold a key (m1 = 0: none)
    const uint32_t wmax = wave_max_u32(m1), wmin = wave_min_u32(m1 ? m1 : 0xFFFFFFFFu);
    if (lane == 0) {
      red_max[wave] = wmax;
      red_min[wave] = wmin;
    }
    if (tid == 0) {
      ncand = 0;
      info[0] = -1;
    }
  }
  __syncthreads();
  uint32_t M = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    M = max(M, red_max[w]);
    lo = min(lo, red_min[w]);
  }
  uint32_t tlo = kMinKey;
  if (k <= 4 * kThreads && lo < M) {  // (uniform)
    // every counted value lies in [lo, M], so the bits above the highest bit in
    // which lo and M differ are common to all of them
    const int hi = 31 - __clz(lo ^ M);
    const int s = hi >= 10 ? hi - 10 : 0;
    const uint32_t dm = (1u << (hi - s + 1)) - 1u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sm[e] >= lo) atomicAdd(&hist[(sm[e] >> s) & dm], 1);
    __syncthreads();
    if (wave == 0) find_bin(hist, (int)dm + 1, k, info);
    __syncthreads();
    if (info[0] >= 0) {  // else fewer than k values were counted: no bound
      const uint32_t pm = hi >= 31 ? 0u : (0xFFFFFFFFu << (hi + 1));
      tlo = (M & pm) | ((uint32_t)info[0] << s);
    }
  }
  tlo = max(tlo, kMinKey);

  // ---- 2. position-ordered count of the live keys; list them in LDS if they fit.
  // A lane's count in a group is at most 4, so a wavefront's sum fits 10 bits:
  // three groups share one prefix sum, in 10-bit fields.
  constexpr int NW = (G + 2) / 3;
  uint32_t lex[G];  // exclusive prefix of this lane's live count in its (group, wave)
  {
    uint32_t packed[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) packed[w] = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t cnt = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += key[4 * g + e] >= tlo ? 1u : 0u;
      packed[g / 3] += cnt << (10 * (g % 3));
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t incl = wave_incl_scan(packed[w]);
#pragma unroll
      for (int q = 0; q < 3 && 3 * w + q < G; ++q) {
        const int g = 3 * w + q;
        const uint32_t fi = (incl >> (10 * q)) & 1023u, fc = (packed[w] >> (10 * q)) & 1023u;
        lex[g] = fi - fc;
        if (lane == 63) tab[g * kWaves + wave] = fi;
      }
    }
  }
  __syncthreads();
  uint32_t goff[G], ltot;
  table_offsets<G>(tab, __builtin_amdgcn_readfirstlane(wave), goff, ltot);
  const int L = (int)ltot;
  const bool in_lds = L <= kListMax;
  if (in_lds) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int at = (int)(goff[g] + lex[g]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key[4 * g + e] >= tlo) {  // (at < L <= kListMax)
          lkey[at] = key[4 * g + e];
          lpos[at] = li_of(g, e);
          ++at;
        }
    }
  }
  // list items of this thread in list mode: [i0, i1), contiguous, in position order
  const int per = (L + kThreads - 1) / kThreads;
  const int i0 = min(L, tid * per), i1 = min(L, i0 + per);

  // ---- 3. radix search for tau among the live keys
  uint32_t prefix, pmask;
  int rem = k;
  for (int b = tid; b < 2048; b += kThreads) hist[b] = 0;
  __syncthreads();  // (also orders the list writes before the list reads)
  if (tlo >= M) {  // every live key equals the maximum
    prefix = M;
    pmask = 0xFFFFFFFFu;
  } else {
    const int hi = 31 - __clz(tlo ^ M);
    int s = hi >= 10 ? hi - 10 : 0;
    int nb = hi - s + 1;
    // bits above `hi` are common to every live key
    pmask = hi >= 31 ? 0u : (0xFFFFFFFFu << (hi + 1));
    prefix = M & pmask;
    bool first = true;
    while (true) {  // uniform
      const uint32_t dm = (1u << nb) - 1u;
      if (!first) {
        for (int b = tid; b < (1 << nb); b += kThreads) hist[b] = 0;
        __syncthreads();
      }
      if (in_lds) {
        for (int i = i0; i < i1; ++i) {
          const uint32_t kv = lkey[i];
          if ((kv & pmask) == prefix) atomicAdd(&hist[(kv >> s) & dm], 1);
        }
      } else {
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (key[j] >= tlo && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> s) & dm], 1);
      }
      __syncthreads();
      if (wave == 0) find_bin(hist, 1 << nb, rem, info);
      __syncthreads();
      const int bsel = info[0], hb = info[2];
      rem -= info[1];
      prefix |= (uint32_t)bsel << s;
      pmask |= dm << s;
      if (hb == rem || s == 0) break;  // the whole bin is selected, or tau is found
      if (in_lds && hb <= kRankMax) {
        // few keys share the boundary bin: gather them (into the histogram's
        // space, free now) and rank each against the others; the key with
        // gt < rem <= ge keys above or equal to it within the bin is tau
        uint32_t* cand = reinterpret_cast<uint32_t*>(hist);
        for (int i = i0; i < i1; ++i) {
          const uint32_t kv = lkey[i];
          if ((kv & pmask) == prefix) {
            const int at = atomicAdd(&ncand, 1);
            if (at < kRankMax) cand[at] = kv;
          }
        }
        __syncthreads();
        if (tid < hb) {
          const uint32_t kv = cand[tid];
          int gt = 0, ge = 0;
          for (int j = 0; j < hb; ++j) {
            const uint32_t o = cand[j];
            gt += o > kv ? 1 : 0;
            ge += o >= kv ? 1 : 0;
          }
          if (gt < rem && rem <= ge) {  // (equal keys agree on both values)
            tau_key = kv;
            tau_gt = gt;
          }
        }
        __syncthreads();
        prefix = tau_key;
        pmask = 0xFFFFFFFFu;
        rem -= tau_gt;
        break;
      }
      const int ns = s >= 11 ? s - 11 : 0;
      nb = s - ns;
      s = ns;
      first = false;
    }
  }

  // ---- 4. emit: keys above the threshold, then the first `rem` keys equal to it;
  // a key's output slot is (# greater before it) + min(# equal before it, rem).
  // Counts are packed as greater | equal << 16 (each below 2^16).
  if (in_lds) {
    uint32_t cnt = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t mk = lkey[i] & pmask;
      cnt += mk > prefix ? 1u : (mk == prefix ? (1u << 16) : 0u);
    }
    const uint32_t incl = wave_incl_scan(cnt);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t before = incl - cnt;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    int gtb = (int)(before & 0xFFFFu), eqb = (int)(before >> 16);
    for (int i = i0; i < i1; ++i) {
      const uint32_t kv = lkey[i], mk = kv & pmask;
      if (mk > prefix) {
        emit(gtb + min(eqb, rem), lpos[i], kv);
        ++gtb;
      } else if (mk == prefix) {
        if (eqb < rem) emit(gtb + eqb, lpos[i], kv);
        ++eqb;
      }
    }
  } else {
    uint32_t gex[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t cnt = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kv = key[4 * g + e], mk = kv & pmask;
        const bool live = kv >= tlo;
        cnt += live && mk > prefix ? 1u : (live && mk == prefix ? (1u << 16) : 0u);
      }
      const uint32_t incl = wave_incl_scan(cnt);
      gex[g] = incl - cnt;
      if (lane == 63) tab[g * kWaves + wave] = incl;
    }
    __syncthreads();
    if (wave == 0) scan_table(tab, E, &total);
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t before = tab[g * kWaves + wave] + gex[g];
      int gtb = (int)(before & 0xFFFFu), eqb = (int)(before >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kv = key[4 * g + e], mk = kv & pmask;
        if (kv < tlo) continue;
        if (mk > prefix) {
          emit(gtb + min(eqb, rem), li_of(g, e), kv);
          ++gtb;
        } else if (mk == prefix) {
          if (eqb < rem) emit(gtb + eqb, li_of(g, e), kv);
          ++eqb;
        }
      }
    }
  }
  finish_slots();
}

// Slots of arbitrary index lists: one thread per entry of the flattened [rows][k]
// list, grid-strided.
__global__ __launch_bounds__(256) void translate_kernel(const int32_t* __restrict__ idx, int64_t ld_idx,
                                                        int64_t rows, int k, SlotMap map) {
  const int64_t total = rows * k;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / k, j = e - r * k;
    map.slots[r * map.ld + j] = physical_slot(map, r, idx[r * ld_idx + j]);
  }
}

// The same with four consecutive entries per thread (one 16-byte index load, two
// 16-byte slot stores, four independent table gathers), for k and both strides
// multiples of four and 16-byte aligned lists.
__global__ __launch_bounds__(256) void translate4_kernel(const int32_t* __restrict__ idx, int64_t ld_idx,
                                                         int64_t rows, int k, SlotMap map) {
  const int q = k / 4;
  const int64_t total = rows * q;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / q, j = 4 * (e - r * q);
    const int4 v = *reinterpret_cast<const int4*>(idx + r * ld_idx + j);
    longlong2* o = reinterpret_cast<longlong2*>(map.slots + r * map.ld + j);
    o[0] = make_longlong2(physical_slot(map, r, v.x), physical_slot(map, r, v.y));
    o[1] = make_longlong2(physical_slot(map, r, v.z), physical_slot(map, r, v.w));
  }
}

template <bool kFirst, bool kLast>
hipError_t launch_level(int R, dim3 grid, hipStream_t s, const float* scores, int64_t ld,
                        Lists src, Lists dst, const int32_t* row_len, int max_row_len, int k,
                        int nlevel, LevelChunks chunks, int32_t* out_idx, float* out_scores,
                        const SlotMap& map, int vec) {
#define DSA_TOPK_CASE(RR)                                                                             \
  case RR:                                                                                            \
    if (vec || !kFirst)                                                                               \
      hipLaunchKernelGGL((topk_level_kernel<RR, kFirst, kLast, true>), grid, dim3(kThreads), 0, s,    \
                         scores, ld, src, dst, row_len, max_row_len, k, nlevel, chunks, out_idx,      \
                         out_scores, map);                                                            \
    else                                                                                              \
      hipLaunchKernelGGL((topk_level_kernel<RR, kFirst, kLast, !kFirst>), grid, dim3(kThreads), 0, s, \
                         scores, ld, src, dst, row_len, max_row_len, k, nlevel, chunks, out_idx,      \
                         out_scores, map);                                                            \
    break;
  switch (R) {
    DSA_TOPK_CASE(4)
    DSA_TOPK_CASE(8)
    DSA_TOPK_CASE(16)
    DSA_TOPK_CASE(24)
    DSA_TOPK_CASE(32)
    DSA_TOPK_CASE(36)
    default:
      return hipErrorInvalidValue;
  }
#undef DSA_TOPK_CASE
  return hipGetLastError();
}

// Plan of levels for rows of up to max_row_len elements.  chunk[l] is the chunk
// size of level l; the last level has a single chunk.
struct Plan {
  int levels = 0;
  int64_t chunk[kMaxLevels];
  int64_t len[kMaxLevels + 1];  // worst-case list length entering level l
};

int pick_r(int64_t n) {
  for (int R : {4, 8, 16, 24, 32, 36})
    if ((int64_t)R * kThreads >= n) return R;
  return kMaxR;
}

// Plan whose first reducing level uses chunks of `first` elements (at least 2k).
Plan plan_with(int max_row_len, int k, int64_t first) {
  Plan p;
  int64_t n = max_row_len;
  p.len[0] = n;
  while (n > kMaxSingle && p.levels < kMaxLevels - 1) {  // (the bound never binds: see kMaxLevels)
    // later levels: chunks of 8k (a power of two, at most 32,768), so a level keeps 1
    // in 8 and still spreads a few long rows over many workgroups
    int64_t C;
    if (p.levels == 0) {
      C = first;
      while (C < 2LL * k) C *= 2;  // each level must shrink the list
    } else {
      C = 4096;
      while (C < 8LL * k && C < kLevelNChunk) C *= 2;  // (C >= 2k for k <= 8192)
    }
    p.chunk[p.levels] = C;
    n = after_level(n, C, k);
    ++p.levels;
    p.len[p.levels] = n;
  }
  p.chunk[p.levels] = (int64_t)pick_r(n) * kThreads;
  ++p.levels;
  return p;
}

// First level of 16,384-element chunks; 32,768 where that saves a whole level (rows
// of 1M keys at k = 1024: 3 levels -> 2, 30.5 -> 28.4 us for 4 such rows), since a
// level's launch and fixed phases cost more than the longer chunks.  Where it saves
// none (16 rows of 131,072: 2 levels either way) the shorter chunks, twice the
// workgroups, are faster (19.3 against 21.5 us).
Plan make_plan(int max_row_len, int k) {
  const Plan a = plan_with(max_row_len, k, kLevel0Chunk);
  if (a.levels <= 2) return a;
  const Plan b = plan_with(max_row_len, k, 2 * kLevel0Chunk);
  return b.levels < a.levels ? b : a;
}

// list row stride: the longest list, rounded up to whole 16-byte loads
int64_t list_cap(const Plan& p) { return (p.len[1] + 3) / 4 * 4; }

}  // namespace

// workspace: two ping-pong candidate lists (none for rows that fit one chunk)
size_t topk_ws_bytes(int rows, int max_row_len, int k) {
  const Plan p = make_plan(max_row_len, k);
  if (p.levels == 1) return 0;
  const int64_t cap = list_cap(p);
  const size_t list = (size_t)rows * (size_t)cap * 8;
  return 2 * ((list + 255) / 256 * 256);
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_len, int rows,
                       int max_row_len, int k, int32_t* out_idx, float* out_scores,
                       const SlotMap& map, void* ws, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const Plan p = make_plan(max_row_len, k);
  Lists none{nullptr, nullptr, 0};
  LevelChunks chunks{};
  for (int l = 0; l < p.levels; ++l) chunks.c[l] = p.chunk[l];
  // 16-byte loads of score rows when every row start is 16-byte aligned
  const int vec = (ld % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) ? 1 : 0;
  if (p.levels == 1) {
    const int R = (int)(p.chunk[0] / kThreads);
    return launch_level<true, true>(R, dim3(1, rows), s, scores, ld, none, none, row_len,
                                    max_row_len, k, 0, chunks, out_idx, out_scores, map, vec);
  }
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  const int64_t cap = list_cap(p);
  const size_t list = ((size_t)rows * (size_t)cap * 8 + 255) / 256 * 256;
  Lists L[2];
  for (int i = 0; i < 2; ++i) {
    uint8_t* b = w8 + i * list;
    L[i] = Lists{reinterpret_cast<uint32_t*>(b), reinterpret_cast<int32_t*>(b + (size_t)rows * cap * 4), cap};
  }
  hipError_t e = hipSuccess;
  for (int l = 0; l < p.levels; ++l) {
    const int64_t C = p.chunk[l];
    const int R = (int)(C / kThreads);
    const unsigned nchunks = (unsigned)((p.len[l] + C - 1) / C);
    const bool first = l == 0, last = l == p.levels - 1;
    const Lists src = first ? none : L[(l - 1) & 1];
    const Lists dst = last ? none : L[l & 1];
    if (first)
      e = launch_level<true, false>(R, dim3(nchunks, rows), s, scores, ld, src, dst, row_len,
                                    max_row_len, k, 0, chunks, out_idx, out_scores, map, vec);
    else if (!last)
      e = launch_level<false, false>(R, dim3(nchunks, rows), s, scores, ld, src, dst, row_len,
                                     max_row_len, k, l, chunks, out_idx, out_scores, map, 1);
    else
      e = launch_level<false, true>(R, dim3(1, rows), s, scores, ld, src, dst, row_len,
                                    max_row_len, k, l, chunks, out_idx, out_scores, map, 1);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_translate(const int32_t* idx, int64_t ld_idx, int rows, int k, const SlotMap& map,
                            hipStream_t s) {
  const int64_t total = (int64_t)rows * k;
  if (total == 0) return hipSuccess;
  const bool quad = k % 4 == 0 && ld_idx % 4 == 0 && map.ld % 2 == 0 &&
                    (reinterpret_cast<uintptr_t>(idx) & 15) == 0 && (reinterpret_cast<uintptr_t>(map.slots) & 15) == 0;
  if (quad) {
    const int64_t blocks = std::min<int64_t>((total / 4 + 255) / 256, 1 << 16);
    hipLaunchKernelGGL(translate4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, idx, ld_idx, (int64_t)rows, k,
                       map);
    return hipGetLastError();
  }
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 1 << 16);
  hipLaunchKernelGGL(translate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, idx, ld_idx, (int64_t)rows, k,
                     map);
  return hipGetLastError();
}

}  // namespace dsa
