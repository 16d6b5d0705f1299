// Internal launchers: host functions, one per kernel family, called by the C ABI
// layer after it has validated every argument.  Each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct KCache {
  uint8_t* base;
  int dtype;       // 1 bf16, 2 fp8
  int block_size;  // 32 or 64
  int64_t num_blocks;
};

struct Rows {
  const int32_t* block_table;
  int max_blocks;
  int num_seqs;
  const int32_t* row_seq;
  const int32_t* row_len;
  int rows;
  int max_row_len;
};

hipError_t launch_store(const uint16_t* x, int64_t n, const int32_t* pos, const int64_t* slots,
                        const KCache& c, uint32_t flags, float eps, float rope_base, int rope_dim,
                        float* dbg, hipStream_t s);

// query preparation: chain flags as for the store, all heads of a row at pos[row]
hipError_t launch_q_prep(const uint16_t* x, int64_t n_vec, int heads, const int32_t* pos, uint32_t flags,
                         float eps, float rope_base, int rope_dim, uint16_t* out_bf16, uint8_t* codes,
                         float* scales, float* dbg, hipStream_t s);
hipError_t launch_quant_fp8(const uint16_t* x, int64_t n_vec, uint8_t* codes, float* scales,
                            hipStream_t s);

// bf16 queries against bf16 or fp8 keys (one query row per workgroup chunk; heads on
// the MFMA M dimension).  write_pad: also write -inf in [row_len, max_row_len).
hipError_t launch_score_decode(const uint16_t* q, const float* w, const KCache& c, const Rows& r,
                               float* scores, int64_t ld, bool write_pad, hipStream_t s);

// fp8 queries against fp8 keys (query tokens x heads on the MFMA M dimension).
hipError_t launch_score_prefill(const uint8_t* q, const float* q_scale, const float* w,
                                const KCache& c, const Rows& r, float* scores, int64_t ld,
                                bool write_pad, hipStream_t s);

// Logical key position -> physical cache slot of a row's selections: the row's
// sequence, visible length and block table, the cache geometry, and where the slots
// go (slots == nullptr: no translation).
struct SlotMap {
  const int32_t* block_table;
  const int32_t* row_seq;
  const int32_t* row_len;
  int max_blocks;
  int num_seqs;
  int block_size;
  int max_row_len;
  int64_t num_blocks;
  int64_t* slots;
  int64_t ld;
};

// top-k over fp32 score rows; ws of topk_ws_bytes(rows, max_row_len, k) bytes.  The
// last level also writes the physical slot of every selection when map.slots is set.
size_t topk_ws_bytes(int rows, int max_row_len, int k);
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* row_len, int rows,
                       int max_row_len, int k, int32_t* out_idx, float* out_scores,
                       const SlotMap& map, void* ws, hipStream_t s);

// physical slots of arbitrary index lists idx [rows][ld_idx] (first k of each row)
hipError_t launch_translate(const int32_t* idx, int64_t ld_idx, int rows, int k, const SlotMap& map,
                            hipStream_t s);

// sparse attention of bf16 query heads [rows][heads][512] over the listed slots of a
// bf16 KV array [num_slots][512]; ws of attention_ws_bytes(rows, k, heads) bytes
size_t attention_ws_bytes(int rows, int k, int heads);
hipError_t launch_attention(const uint16_t* q, int heads, const uint8_t* kv, int64_t num_slots, const int64_t* slots,
                            int64_t ld, int k, int rows, float scale, float* out, float* lse, void* ws,
                            hipStream_t s);

}  // namespace dsa
