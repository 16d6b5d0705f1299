// Decode scoring: one bf16 query row (64 index heads x 128) against the paged
// index-K cache (bf16 keys, fp8 e4m3 keys with a per-token fp32 scale, or MXFP4 keys:
// e2m1 codes with an e8m0 scale per 32 dims):
//     score[p] = s_p * sum_h w_h * max(0, q_h . k_p)
// (the lightning-indexer q.k score of ROCm/ATOM issue 1507, "Root cause found"; the
// paged read through the block table is the analog of the pages'
// deepgemm_fp8_paged_mqa_logits, "How it was isolated").
//
// Design for gfx950:
//  - All 64 heads of a row share every key (multi-query), so each 16-key group is a
//    dense [64 x 128] . [128 x 16] product: four 16-head M tiles x four K=32 steps of
//    v_mfma_f32_16x16x32_bf16.  At ~8 TB/s of fp8 keys the contraction needs
//    ~0.5 P MAC/s, far beyond the vector ALU, so it must run on the matrix cores.
//  - Each wavefront holds the whole query row as MFMA A operands in registers
//    (64 VGPRs) and scores its own keys: no cross-wave reduction.  The row (16 KB)
//    is copied into LDS once per workgroup and read from there by every wave.  bf16
//    and fp8 keys use the plain MFMA operand order (K-step s, lane row g: dims
//    32*s + 8*g .. +7).
//  - Keys of every format stream through a per-wave LDS ring filled by LDS DMA
//    (score_decode_ring_kernel), which keeps several 16-key groups in flight
//    without holding VGPRs.
//  - fp8 codes are widened to bf16 exactly (every e4m3 value is a bf16 value) with
//    v_cvt_scalef32_pk_bf16_fp8; the per-key scale multiplies the head sum.
//  - MXFP4: lane l's 32 contiguous dims 32*(l/16) .. +31 are exactly one 32-element
//    scale block of its key, so the lane widens its 16 code bytes with
//    v_cvt_scalef32_pk_bf16_fp4 and the block's power-of-two scale folded in
//    (e2m1 * 2^k is a bf16 value; the conversion uses the scale's exponent, and
//    reproduces every e2m1 * 2^k for k in [-127, 121] exactly on the hardware).
//  - The ReLU-weighted head sum is in-lane (16 of the 64 heads per lane) plus two
//    cross-lane adds; lane l ends up with the score of key l%16 of its group, and
//    64 scores at a time leave with one coalesced 256-byte write.
#include "common.hpp"
#include "launch.hpp"

namespace dsa {
namespace {

constexpr int kSpan = 64;  // keys per span (one 64-token block, or two 32-token blocks)
constexpr int kQRowBytes = 64 * kHeadDim * 2;  // one bf16 query row

enum KeyKind { kBf16Keys = 0, kFp8Keys = 1, kFp4Keys = 2 };

__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  union {
    bf16x2_t h[4];
    bf16x8_t v;
  } u;
  u.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false);
  u.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true);
  u.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false);
  u.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true);
  return u.v;
}

// 8 e2m1 codes (element 2i in the low nibble of byte i) -> 8 bf16 values, times the
// power-of-two scale
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t d, float scale) {
  union {
    bf16x2_t h[4];
    bf16x8_t v;
  } u;
  u.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0);
  u.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1);
  u.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2);
  u.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3);
  return u.v;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  union {
    uint4 u;
    bf16x8_t b;
  } x;
  x.u = v;
  return x.b;
}

// ---------------------------------------------------------------------------
// The key stream goes through LDS DMA.  Each wave owns a ring of kRing 16-key group
// slots in LDS and keeps kRing-1 groups in flight with global_load_lds (no VGPRs
// held by loads in flight), so far more bytes are outstanding per wave than a
// register double buffer allows (bf16 spans held in registers took 232 VGPRs, 2
// waves per SIMD).  Every group issues a fixed number of loads (fp8: 2 x 1 KB of
// codes and 64 B of scales; MXFP4: 1 KB of codes and 64 B of e8m0 scales; bf16:
// 4 x 1 KB), so a fixed vmcnt wait guarantees the group about to be read has
// landed; the score stores interleaved with the loads only make that wait
// stricter.  Within a slot, 16-byte chunks are XOR-swizzled by key so a read phase
// (several keys, same chunk) hits distinct banks: fp8 chunk c of key r sits at
// position r*8 + (c ^ ((r >> 1) & 7)), MXFP4 chunk c at r*4 + (c ^ ((r >> 2) & 3)),
// bf16 chunk c at r*16 + (c ^ r).
#ifndef DSA_DECODE_RING
#define DSA_DECODE_RING 3
#endif
#ifndef DSA_DECODE_RING4
#define DSA_DECODE_RING4 6
#endif
#ifndef DSA_DECODE_RING16
#define DSA_DECODE_RING16 3
#endif
constexpr int kDecodeRing = DSA_DECODE_RING;      // LDS slots per wave, fp8 keys
constexpr int kDecodeRing4 = DSA_DECODE_RING4;    // MXFP4 keys (smaller slots, deeper ring)
constexpr int kDecodeRing16 = DSA_DECODE_RING16;  // bf16 keys (4 KB slots)

template <int kKind>
struct RingKeys {
  static constexpr bool kFp4 = kKind == kFp4Keys, kBf16 = kKind == kBf16Keys;
  static constexpr int kRow = kBf16 ? 256 : (kFp4 ? 64 : 128);  // key bytes before the scales
  static constexpr int kCodes = 16 * kRow;                         // code bytes of a group
  static constexpr int kSlot = kCodes + (kBf16 ? 0 : 16 * 4);      // + the 16 keys' scale words
                                                                   // (fp8 2112, MXFP4 1088, bf16 4096 bytes)
  static constexpr int kKeyBytes = kBf16 ? 256 : (kFp4 ? 68 : 132);  // cache bytes per token
  static constexpr int kLoads = kBf16 ? 4 : (kFp4 ? 2 : 3);          // load instructions per group
};

// Every key group is read once.  fp8 and bf16 groups are loaded with the
// non-temporal cache policy (NT), which leaves L2 to the query rows and block
// tables: measured 8% faster on decode batch 32 with fp8 keys, 4% on 16 x 128k fp8
// keys and 12% on 16 x 128k bf16 keys.  MXFP4 groups, at half the bytes, measured
// no gain and keep the default policy.
template <int BS, int kKind>
__device__ __forceinline__ void issue_group(uint8_t* slot, const uint8_t* cache, int phys, int p0, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
  using K = RingKeys<kKind>;
  constexpr int kCpol = K::kFp4 ? 0 : 2;  // cache policy bits of the loads: 2 = NT
  const uint8_t* blk = cache + (int64_t)phys * (BS * K::kKeyBytes);
  const int off = p0 % BS;
  if constexpr (K::kBf16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sidx = j * 64 + lane, r = sidx >> 4, c = (sidx & 15) ^ r;
      __builtin_amdgcn_global_load_lds(blk + (off + r) * 256 + c * 16,
                                       (lds_void*)(slot + j * 1024), 16, 0, kCpol);
    }
    return;  // (no scales)
  } else if constexpr (K::kFp4) {
    const int r = lane >> 2, c = (lane & 3) ^ ((r >> 2) & 3);
    __builtin_amdgcn_global_load_lds(blk + (off + r) * 64 + c * 16, (lds_void*)slot, 16, 0, kCpol);
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int sidx = j * 64 + lane, r = sidx >> 3, c = (sidx & 7) ^ ((r >> 1) & 7);
      __builtin_amdgcn_global_load_lds(blk + (off + r) * 128 + c * 16,
                                       (lds_void*)(slot + j * 1024), 16, 0, kCpol);
    }
  }
  if (lane < 16)  // the 16 keys' scale words (fp32, or four e8m0 bytes)
    __builtin_amdgcn_global_load_lds(blk + BS * K::kRow + (off + lane) * 4,
                                     (lds_void*)(slot + K::kCodes), 4, 0, kCpol);
}

template <int BS, int kRing, int kKind>
__global__ __launch_bounds__(256, 2) void score_decode_ring_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ cache,
    int64_t num_blocks, const int32_t* __restrict__ block_table, int max_blocks, int num_seqs,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_len, int max_row_len,
    float* __restrict__ scores, int64_t ld, int spans_per_wave, int write_pad) {
  // ring[slot][wave]: slot s of the four waves is contiguous, so slots 1 .. kRing-1
  // together hold the 16 KB query row while it is staged (they are free until the
  // wave issues its second group)
  constexpr bool kFp4 = RingKeys<kKind>::kFp4, kBf16 = RingKeys<kKind>::kBf16;
  constexpr int kSlot = RingKeys<kKind>::kSlot;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][4][kSlot];
  static_assert((kRing - 1) * 4 * kSlot >= kQRowBytes + 256, "query row and weights fit the staging slots");
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = blockIdx.y;
  const int seq = row_seq[r];
  const int n = min(max(row_len[r], 0), max_row_len);
  float* out = scores + (int64_t)r * ld;
  const int chunk0 = blockIdx.x * (4 * spans_per_wave * kSpan);
  const bool seq_bad = seq < 0 || seq >= num_seqs;

  if (chunk0 >= n || seq_bad) {  // nothing to read: padding, or NaN for a bad sequence
    const int end = min(chunk0 + 4 * spans_per_wave * kSpan, max_row_len);
    for (int p = chunk0 + (int)threadIdx.x; p < end; p += 256) {
      if (p < n) out[p] = __builtin_nanf("");
      else if (write_pad) out[p] = -INFINITY;
    }
    return;
  }
  const int32_t* bt_row = block_table + (int64_t)seq * max_blocks;
  // this wave's spans: chunk0 + (i*4 + wave)*64, i < spans_per_wave; groups t = 4i + g
  auto group_pos = [&](int t) { return chunk0 + ((t >> 2) * 4 + wave) * kSpan + 16 * (t & 3); };
  int ngroups = 0;  // the real groups are a prefix: positions grow with t
  while (ngroups < 4 * spans_per_wave && group_pos(ngroups) < n) ++ngroups;

  // lane j holds the physical block of group j; block 0 stands in for a bad entry
  // (whose scores become NaN) and for groups past the wave's work (loaded, never read)
  int my_phys = 0;
  bool my_bad = false;
  if (lane < ngroups) {
    const int ph = bt_row[group_pos(lane) / BS];
    my_bad = ph < 0 || ph >= num_blocks;
    my_phys = my_bad ? 0 : ph;
  }
  const uint64_t bad_groups = __ballot(my_bad);

  auto my = [&](int slot) { return &ring[slot][wave][0]; };

  // The query row goes to LDS once per workgroup (each wave copies 16 heads with LDS
  // DMA) instead of once per wave: every wave needs all 16 KB of it as A operands,
  // and four separate copies from L2 had cost more than all the MFMA work.  Chunk c
  // (16 bytes) of head h sits at position c ^ (h % 16) of the head's 256 bytes, so
  // the eight lanes of a 16-byte read phase (eight heads, one chunk) hit distinct
  // banks.  The copy is issued before group 0, so waiting for it leaves group 0 in
  // flight.
  // The head weights (256 bytes) follow the query row in the staging slots, copied
  // by wave 0.  (Loaded into registers directly, they would be the only loads the
  // compiler tracks, and it would wait for every load, the key groups included,
  // before the first group.)
  uint8_t* qs = &ring[1][0][0];
  {
    typedef __attribute__((address_space(3))) void lds_void;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q) + (int64_t)r * 64 * kHeadDim * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int P = (wave * 4 + j) * 1024 + lane * 16, h = P >> 8;
      const int c = ((P >> 4) & 15) ^ (h & 15);
      __builtin_amdgcn_global_load_lds(qrow + h * 256 + c * 16, (lds_void*)(qs + (wave * 4 + j) * 1024), 16, 0, 0);
    }
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(w + (int64_t)r * 64 + lane, (lds_void*)(qs + kQRowBytes), 4, 0, 0);
  }
  issue_group<BS, kKind>(my(0), cache, __builtin_amdgcn_readlane(my_phys, 0), group_pos(0), lane);
  // every wave's share landed (group 0's loads may stay in flight)
  __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(RingKeys<kKind>::kLoads) : "memory");

  // A operands: K-step s4 of M tile mt holds head 16*mt + lane%16 and, for fp8 and
  // bf16 keys, dims 32*s4 + 8*(lane/16) .. +7 (chunk 4*s4 + lane/16, the plain MFMA
  // order); for
  // MXFP4 keys, whose lane keeps one whole 32-dim scale block, dims 32*(lane/16) +
  // 8*s4 .. +7 (chunk 4*(lane/16) + s4)
  // wv: weights of the accumulator rows this lane holds, head 16*mt + 4*(lane/16) + v
  bf16x8_t qa[4][4];
  float wv[4][4];
  {
    const uint32_t qb = (uint32_t)(uintptr_t)qs;
    const int hl = lane & 15, g4 = lane >> 4;
    auto qchunk = [&](int s4) { return kFp4 ? 4 * g4 + s4 : 4 * s4 + g4; };
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t hb = qb + (16 * mt + hl) * 256;
      uint4 x0, x1, x2, x3;
      float4 wq;
      __asm__ volatile(
          "ds_read_b128 %0, %5\n\t"
          "ds_read_b128 %1, %6\n\t"
          "ds_read_b128 %2, %7\n\t"
          "ds_read_b128 %3, %8\n\t"
          "ds_read_b128 %4, %9\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(wq)
          : "v"(hb + ((qchunk(0) ^ hl) << 4)), "v"(hb + ((qchunk(1) ^ hl) << 4)),
            "v"(hb + ((qchunk(2) ^ hl) << 4)), "v"(hb + ((qchunk(3) ^ hl) << 4)),
            "v"(qb + kQRowBytes + (16 * mt + 4 * g4) * 4)
          : "memory");
      qa[mt][0] = as_bf16x8(x0);
      qa[mt][1] = as_bf16x8(x1);
      qa[mt][2] = as_bf16x8(x2);
      qa[mt][3] = as_bf16x8(x3);
      wv[mt][0] = wq.x;
      wv[mt][1] = wq.y;
      wv[mt][2] = wq.z;
      wv[mt][3] = wq.w;
    }
  }
  __asm__ volatile("s_barrier" ::: "memory");  // every wave has its operands: the slots are free
#pragma unroll
  for (int t = 1; t < kRing - 1; ++t)
    issue_group<BS, kKind>(my(t), cache, __builtin_amdgcn_readlane(my_phys, t), group_pos(t), lane);

  // read positions of this lane in a slot: key lane%16; fp8: dims 32*s4 + 8*(lane/16)
  // .. +7, i.e. half (lane/16)&1 of code chunk 2*s4 + lane/32; MXFP4: code chunk
  // lane/16 (dims 32*(lane/16) .. +31) and scale byte lane/16 of the key's word;
  // bf16: one 16-byte chunk per K-step
  const int kr = lane & 15;
  const int g4 = lane >> 4;
  int rd[4];
  if constexpr (kBf16) {  // chunk 4*s4 + lane/16 of key kr (dims 32*s4 + 8*(lane/16) .. +7)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) rd[s4] = kr * 256 + (((4 * s4 + g4) ^ kr) << 4);
  } else if constexpr (kFp4) {
    rd[0] = kr * 64 + ((g4 ^ ((kr >> 2) & 3)) << 4);
    rd[1] = rd[2] = rd[3] = rd[0];
  } else {
    const int sw = (kr >> 1) & 7;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) rd[s4] = kr * 128 + (((2 * s4 + (g4 >> 1)) ^ sw) << 4) + 8 * (g4 & 1);
  }

  float val = 0.0f;
  uint32_t bad = 0;  // bit g: group g of the current span lies in a bad block
  int wslot = kRing - 1, rslot = 0;
  for (int t = 0; t < ngroups; ++t) {
    const int tn = t + kRing - 1;  // (readlane of a lane >= ngroups gives block 0)
    issue_group<BS, kKind>(my(wslot), cache, __builtin_amdgcn_readlane(my_phys, tn & 63), group_pos(tn), lane);
    wslot = wslot == kRing - 1 ? 0 : wslot + 1;
    // wait for group t (the kLoads loads of each of the kRing - 1 newer groups may
    // stay in flight), then read this lane's operands and its key's scale; the waits
    // sit in the asm because the compiler would otherwise drain every load before any
    // LDS read
    const uint32_t sbase = (uint32_t)(uintptr_t)my(rslot);
    rslot = rslot == kRing - 1 ? 0 : rslot + 1;
    // the slot's codes: fp8, four 8-byte halves (one per K-step); MXFP4, one 16-byte
    // chunk (one dword per K-step) and the key's four e8m0 bytes
    uint2 c[4];
    uint4 cb[4];  // bf16 keys: the four K-steps' 16-byte operands
    float ks;     // the key's scale (fp8), or 1 (MXFP4: the block scale is in the B operand)
    float bscale = 1.0f;
    if constexpr (kBf16) {
      __asm__ volatile(
          "s_waitcnt vmcnt(%8)\n\t"
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(cb[0]), "=&v"(cb[1]), "=&v"(cb[2]), "=&v"(cb[3])
          : "v"(sbase + rd[0]), "v"(sbase + rd[1]), "v"(sbase + rd[2]), "v"(sbase + rd[3]),
            "n"(4 * (kRing - 1))
          : "memory");
      ks = 1.0f;
    } else if constexpr (kFp4) {
      uint4 c4;
      uint32_t sw4;
      __asm__ volatile(
          "s_waitcnt vmcnt(%4)\n\t"
          "ds_read_b128 %0, %2\n\t"
          "ds_read_b32 %1, %3\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(c4), "=&v"(sw4)
          : "v"(sbase + rd[0]), "v"(sbase + RingKeys<kKind>::kCodes + 4 * kr), "n"(2 * (kRing - 1))
          : "memory");
      const uint32_t e8 = (sw4 >> (8 * g4)) & 0xFFu;
      bscale = __uint_as_float(e8 ? e8 << 23 : 0x00400000u);  // 2^(e8-127)
      c[0].x = c4.x;
      c[1].x = c4.y;
      c[2].x = c4.z;
      c[3].x = c4.w;
      ks = 1.0f;
    } else {
      __asm__ volatile(
          "s_waitcnt vmcnt(%10)\n\t"
          "ds_read_b64 %0, %5\n\t"
          "ds_read_b64 %1, %6\n\t"
          "ds_read_b64 %2, %7\n\t"
          "ds_read_b64 %3, %8\n\t"
          "ds_read_b32 %4, %9\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(ks)
          : "v"(sbase + rd[0]), "v"(sbase + rd[1]), "v"(sbase + rd[2]), "v"(sbase + rd[3]),
            "v"(sbase + RingKeys<kKind>::kCodes + 4 * kr), "n"(3 * (kRing - 1))
          : "memory");
    }
    const int p0 = group_pos(t);
    bad |= (uint32_t)((bad_groups >> t) & 1) << (t & 3);
    f32x4_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const bf16x8_t b = kBf16 ? as_bf16x8(cb[s4])
                               : (kFp4 ? fp4x8_to_bf16x8(c[s4].x, bscale) : fp8x8_to_bf16x8(c[s4].x, c[s4].y));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s4], b, acc[mt], 0, 0, 0);
    }
    // fp8 and MXFP4 keys: the group's epilogue stays after all of its MFMAs (left to
    // itself the compiler mixed it into the next group's ring read and widening:
    // decode_b32 16.2 -> 14.1 us; 16 x 131,072 fp8 keys 1-2% faster; bf16 keys were
    // not faster and keep the compiler's order)
    if constexpr (!kBf16) __builtin_amdgcn_sched_barrier(0);
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) part = fmaf(wv[mt][v], relu(acc[mt][v]), part);
    part = rows4_sum(part) * ks;
    if ((lane >> 4) == (t & 3)) val = part + 0.0f;  // +0.0f: a zero score is +0
    if ((t & 3) == 3 || t + 1 == ngroups) {  // end of a span: one coalesced store
      const int p = (p0 & ~(kSpan - 1)) + lane;
      float v = val;
      if ((bad >> (lane >> 4)) & 1u) v = __builtin_nanf("");  // only the bad block's keys
      if (p >= n) v = -INFINITY;
      if (p < max_row_len) out[p] = v;
      val = 0.0f;
      bad = 0;
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the ring before the wave ends
  if (write_pad)  // this wave's spans past the row's keys
    for (int i = 0; i < spans_per_wave; ++i) {
      const int p = chunk0 + (i * 4 + wave) * kSpan + lane;
      if (p - lane >= n && p < max_row_len) out[p] = -INFINITY;
    }
}

template <int kKeys>
hipError_t launch_bs(const uint16_t* q, const float* w, const KCache& c, const Rows& r,
                     float* scores, int64_t ld, bool write_pad, hipStream_t s) {
  const int64_t spans_row = (r.max_row_len + kSpan - 1) / kSpan;
  const int64_t total = spans_row * r.rows;
  // aim for >= ~4 workgroups per CU on the 256-CU part, at most 8 spans per wave
  int spw = (int)(total / (4 * 1024));
  spw = spw < 1 ? 1 : (spw > 8 ? 8 : spw);
#ifdef DSA_DECODE_SPW
  spw = DSA_DECODE_SPW;
#endif
  const int64_t per_wg = 4LL * spw;
  const dim3 grid((unsigned)((spans_row + per_wg - 1) / per_wg), (unsigned)r.rows), block(256);
#define DSA_RING_LAUNCH(BSV, RING, FP4)                                                              \
  hipLaunchKernelGGL((score_decode_ring_kernel<BSV, RING, FP4>), grid, block, 0, s, q, w, c.base,   \
                     c.num_blocks, r.block_table, r.max_blocks, r.num_seqs, r.row_seq, r.row_len, \
                     r.max_row_len, scores, ld, spw, (int)write_pad)
  if constexpr (kKeys == kFp8Keys) {  // fp8 keys: the LDS-ring kernel
    if (c.block_size == 64) DSA_RING_LAUNCH(64, kDecodeRing, kFp8Keys);
    else DSA_RING_LAUNCH(32, kDecodeRing, kFp8Keys);
  } else if constexpr (kKeys == kFp4Keys) {  // MXFP4 keys
    if (c.block_size == 64) DSA_RING_LAUNCH(64, kDecodeRing4, kFp4Keys);
    else DSA_RING_LAUNCH(32, kDecodeRing4, kFp4Keys);
  } else {  // bf16 keys
    if (c.block_size == 64) DSA_RING_LAUNCH(64, kDecodeRing16, kBf16Keys);
    else DSA_RING_LAUNCH(32, kDecodeRing16, kBf16Keys);
  }
#undef DSA_RING_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_decode(const uint16_t* q, const float* w, const KCache& c, const Rows& r,
                               float* scores, int64_t ld, bool write_pad, hipStream_t s) {
  if (r.rows == 0 || r.max_row_len == 0) return hipSuccess;
  if (c.dtype == 2) return launch_bs<kFp8Keys>(q, w, c, r, scores, ld, write_pad, s);
  if (c.dtype == 3) return launch_bs<kFp4Keys>(q, w, c, r, scores, ld, write_pad, s);
  return launch_bs<kBf16Keys>(q, w, c, r, scores, ld, write_pad, s);
}

}  // namespace dsa
