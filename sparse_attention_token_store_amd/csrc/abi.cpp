// C ABI of the indexer library: argument validation on the host (nothing is
// launched unless every check passes), dispatch to the kernel launchers, and the
// thread-local error message.  The validation never calls the HIP runtime, so it
// behaves the same on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "dsa_indexer.h"
#include "launch.hpp"

// Workspace of indexer_score_topk_static: one copy per GPU, from the moment the
// library's code object is loaded on that GPU until the process ends.  On the host
// this name is only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[IDX_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int32_t kMaxK = 8192;
constexpr int32_t kMaxRows = 65535;       // grid y dimension
constexpr int32_t kHeadsV1 = 64;
constexpr int32_t kMaxAttnK = 1 << 16;    // listed slots per attention row

int32_t check_cache(const idx_kcache& c) {
  if (!c.base) return fail(IDX_EINVAL, "cache.base is NULL");
  if (!aligned(c.base, 256)) return fail(IDX_EINVAL, "cache.base must be 256-byte aligned");
  if (c.dtype != IDX_BF16 && c.dtype != IDX_FP8_E4M3 && c.dtype != IDX_MXFP4)
    return fail(IDX_EINVAL, "cache.dtype %d is not IDX_BF16, IDX_FP8_E4M3 or IDX_MXFP4", c.dtype);
  if (c.block_size != 32 && c.block_size != 64)
    return fail(IDX_EUNSUPPORTED, "cache.block_size %d unsupported (32 or 64)", c.block_size);
  if (c.num_blocks < 1) return fail(IDX_EINVAL, "cache.num_blocks must be >= 1");
  if (c.num_blocks > (int64_t)INT32_MAX) return fail(IDX_EINVAL, "cache.num_blocks too large");
  return IDX_OK;
}

int32_t check_rows(const idx_rows& r) {
  if (r.rows < 0 || r.rows > kMaxRows) return fail(IDX_EINVAL, "rows %d out of [0, %d]", r.rows, kMaxRows);
  if (r.max_row_len < 0) return fail(IDX_EINVAL, "max_row_len must be >= 0");
  if (r.rows == 0) return IDX_OK;
  if (!r.block_table || !r.row_seq || !r.row_len)
    return fail(IDX_EINVAL, "block_table, row_seq and row_len must be non-NULL");
  if (r.max_blocks < 1 || r.num_seqs < 1) return fail(IDX_EINVAL, "max_blocks and num_seqs must be >= 1");
  return IDX_OK;
}

int32_t check_score_args(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                         int32_t heads, const idx_kcache& cache, const idx_rows& rows) {
  if (int32_t e = check_cache(cache)) return e;
  if (int32_t e = check_rows(rows)) return e;
  if ((int64_t)rows.max_row_len > (int64_t)rows.max_blocks * cache.block_size)
    return fail(IDX_EINVAL, "max_row_len %d exceeds max_blocks*block_size", rows.max_row_len);
  if (heads != kHeadsV1) return fail(IDX_EUNSUPPORTED, "heads=%d unsupported (64)", heads);
  if (q_dtype != IDX_BF16 && q_dtype != IDX_FP8_E4M3)
    return fail(IDX_EINVAL, "q_dtype %d is not IDX_BF16 or IDX_FP8_E4M3", q_dtype);
  if (q_dtype == IDX_FP8_E4M3 && cache.dtype == IDX_BF16)
    return fail(IDX_EUNSUPPORTED, "fp8 queries against bf16 keys are not supported");
  if (rows.rows == 0) return IDX_OK;
  if (!q || !w) return fail(IDX_EINVAL, "q and w must be non-NULL");
  if (!aligned(q, 16)) return fail(IDX_EINVAL, "q must be 16-byte aligned");
  if (!aligned(w, 4)) return fail(IDX_EINVAL, "w must be 4-byte aligned");
  if (q_dtype == IDX_FP8_E4M3) {
    if (!q_scale) return fail(IDX_EINVAL, "q_scale is required for fp8 queries");
    if (!aligned(q_scale, 4)) return fail(IDX_EINVAL, "q_scale must be 4-byte aligned");
  }
  return IDX_OK;
}

dsa::KCache to_kc(const idx_kcache& c) {
  return dsa::KCache{static_cast<uint8_t*>(c.base), c.dtype, c.block_size, c.num_blocks};
}
dsa::Rows to_rows(const idx_rows& r) {
  return dsa::Rows{r.block_table, r.max_blocks, r.num_seqs, r.row_seq, r.row_len, r.rows, r.max_row_len};
}
dsa::SlotMap to_map(const idx_kcache& c, const idx_rows& r, int64_t* slots, int64_t ld) {
  return dsa::SlotMap{r.block_table, r.row_seq,   r.row_len,    r.max_blocks, r.num_seqs,
                      c.block_size,  r.max_row_len, c.num_blocks, slots,        ld};
}

int32_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(IDX_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return IDX_OK;
}

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// score_topk workspace: the score rows (ld rounded to 64), then the top-k lists
int64_t score_ld(int32_t max_row_len) { return round_up(max_row_len > 0 ? max_row_len : 1, 64); }
size_t score_bytes(int32_t rows, int32_t max_row_len) {
  return (size_t)round_up((int64_t)rows * score_ld(max_row_len) * 4, 256);
}

// Device address of `scratch` on the GPU that owns `s` (the current device for the
// null stream), looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_of_stream(hipStream_t s, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(IDX_ELAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  dev = cur;
  if (s) {
    e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) return fail(IDX_ELAUNCH, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(IDX_EUNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(IDX_ELAUNCH, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return fail(IDX_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return IDX_OK;
}

}  // namespace

#define IDX_API __attribute__((visibility("default")))

extern "C" {

IDX_API int32_t indexer_abi_version(void) { return IDX_ABI_VERSION; }

IDX_API const char* indexer_last_error(void) { return g_err.c_str(); }

IDX_API size_t indexer_workspace_bytes(int32_t op, int32_t rows, int32_t max_row_len, int32_t k) {
  if (rows < 0 || rows > kMaxRows || max_row_len < 0 || k < 1 || k > kMaxK) return 0;
  if (op == IDX_OP_TOPK) return dsa::topk_ws_bytes(rows, max_row_len, k);
  if (op == IDX_OP_SCORE_TOPK)
    return score_bytes(rows, max_row_len) + dsa::topk_ws_bytes(rows, max_row_len, k);
  return 0;
}

IDX_API int32_t index_k_store(const void* x_bf16, int64_t n, const int32_t* positions,
                      const int64_t* slot_mapping, idx_kcache cache, uint32_t flags, float rms_eps,
                      float rope_base, int32_t rope_dim, float* prequant_dbg, void* hip_stream) {
  g_err.clear();
  if (n < 0) return fail(IDX_EINVAL, "n must be >= 0");
  if (flags & ~7u) return fail(IDX_EINVAL, "unknown flag bits 0x%x", flags & ~7u);
  if (int32_t e = check_cache(cache)) return e;
  if (flags & IDX_STORE_ROPE) {
    if (rope_dim < 2 || rope_dim > IDX_HEAD_DIM || (rope_dim & 1))
      return fail(IDX_EINVAL, "rope_dim %d must be even and in [2, 128]", rope_dim);
    if (!(rope_base > 0.0f) || !std::isfinite(rope_base)) return fail(IDX_EINVAL, "rope_base must be finite and > 0");
  }
  if ((flags & IDX_STORE_RMSNORM) && (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps)))
    return fail(IDX_EINVAL, "rms_eps must be finite and >= 0");
  if (n == 0) return IDX_OK;
  if (n > (int64_t)INT32_MAX * 4) return fail(IDX_EINVAL, "n too large");
  if (!x_bf16 || !slot_mapping) return fail(IDX_EINVAL, "x_bf16 and slot_mapping must be non-NULL");
  if (!aligned(x_bf16, 4)) return fail(IDX_EINVAL, "x_bf16 must be 4-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(IDX_EINVAL, "slot_mapping must be 8-byte aligned");
  if ((flags & IDX_STORE_ROPE) && !positions) return fail(IDX_EINVAL, "positions is required with IDX_STORE_ROPE");
  if (positions && !aligned(positions, 4)) return fail(IDX_EINVAL, "positions must be 4-byte aligned");
  if (prequant_dbg && !aligned(prequant_dbg, 8)) return fail(IDX_EINVAL, "prequant_dbg must be 8-byte aligned");
  return launched(dsa::launch_store(static_cast<const uint16_t*>(x_bf16), n, positions, slot_mapping,
                                    to_kc(cache), flags, rms_eps, rope_base, rope_dim, prequant_dbg,
                                    static_cast<hipStream_t>(hip_stream)),
                  "index_k_store");
}

IDX_API int32_t indexer_q_prep(const void* q_bf16, int64_t n_vec, int32_t heads, const int32_t* positions,
                               uint32_t flags, float rms_eps, float rope_base, int32_t rope_dim,
                               void* out_bf16, uint8_t* codes, float* scales, float* prequant_dbg,
                               void* hip_stream) {
  g_err.clear();
  if (n_vec < 0) return fail(IDX_EINVAL, "n_vec must be >= 0");
  if (heads < 1) return fail(IDX_EINVAL, "heads must be >= 1");
  if (n_vec % heads) return fail(IDX_EINVAL, "n_vec %lld is not a multiple of heads %d", (long long)n_vec, heads);
  if (flags & ~7u) return fail(IDX_EINVAL, "unknown flag bits 0x%x", flags & ~7u);
  if (flags & IDX_STORE_ROPE) {
    if (rope_dim < 2 || rope_dim > IDX_HEAD_DIM || (rope_dim & 1))
      return fail(IDX_EINVAL, "rope_dim %d must be even and in [2, 128]", rope_dim);
    if (!(rope_base > 0.0f) || !std::isfinite(rope_base)) return fail(IDX_EINVAL, "rope_base must be finite and > 0");
  }
  if ((flags & IDX_STORE_RMSNORM) && (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps)))
    return fail(IDX_EINVAL, "rms_eps must be finite and >= 0");
  if (n_vec == 0) return IDX_OK;  // nothing to do: outputs of no elements may be NULL
  if ((codes == nullptr) != (scales == nullptr)) return fail(IDX_EINVAL, "codes and scales go together");
  if (!out_bf16 && !codes && !prequant_dbg) return fail(IDX_EINVAL, "no output requested");
  if (n_vec > ((int64_t)1 << 40)) return fail(IDX_EINVAL, "n_vec too large");
  if ((n_vec / heads) * (((int64_t)heads + 3) / 4) > (int64_t)INT32_MAX * 4)
    return fail(IDX_EINVAL, "too many vectors for one launch (rows * ceil(heads / 4) > 4 * INT32_MAX)");
  if (!q_bf16) return fail(IDX_EINVAL, "q_bf16 must be non-NULL");
  // the kernel moves 16-byte chunks of q, out_bf16 and prequant_dbg and 8-byte
  // chunks of codes
  if (!aligned(q_bf16, 16)) return fail(IDX_EINVAL, "q_bf16 must be 16-byte aligned");
  if ((flags & IDX_STORE_ROPE) && !positions) return fail(IDX_EINVAL, "positions is required with IDX_STORE_ROPE");
  if (positions && !aligned(positions, 4)) return fail(IDX_EINVAL, "positions must be 4-byte aligned");
  if (out_bf16 && !aligned(out_bf16, 16)) return fail(IDX_EINVAL, "out_bf16 must be 16-byte aligned");
  if (codes && !aligned(codes, 8)) return fail(IDX_EINVAL, "codes must be 8-byte aligned");
  if (scales && !aligned(scales, 4)) return fail(IDX_EINVAL, "scales must be 4-byte aligned");
  if (prequant_dbg && !aligned(prequant_dbg, 16)) return fail(IDX_EINVAL, "prequant_dbg must be 16-byte aligned");
  return launched(dsa::launch_q_prep(static_cast<const uint16_t*>(q_bf16), n_vec, heads, positions, flags,
                                     rms_eps, rope_base, rope_dim, static_cast<uint16_t*>(out_bf16), codes,
                                     scales, prequant_dbg, static_cast<hipStream_t>(hip_stream)),
                  "indexer_q_prep");
}

IDX_API int32_t indexer_quant_fp8(const void* x_bf16, int64_t n_vec, uint8_t* codes, float* scales,
                          void* hip_stream) {
  g_err.clear();
  if (n_vec < 0) return fail(IDX_EINVAL, "n_vec must be >= 0");
  if (n_vec == 0) return IDX_OK;
  if (n_vec > (int64_t)INT32_MAX * 16) return fail(IDX_EINVAL, "n_vec too large");
  if (!x_bf16 || !codes || !scales) return fail(IDX_EINVAL, "x_bf16, codes and scales must be non-NULL");
  if (!aligned(x_bf16, 16)) return fail(IDX_EINVAL, "x_bf16 must be 16-byte aligned");
  if (!aligned(codes, 8)) return fail(IDX_EINVAL, "codes must be 8-byte aligned");
  if (!aligned(scales, 4)) return fail(IDX_EINVAL, "scales must be 4-byte aligned");
  return launched(dsa::launch_quant_fp8(static_cast<const uint16_t*>(x_bf16), n_vec, codes, scales,
                                        static_cast<hipStream_t>(hip_stream)),
                  "indexer_quant_fp8");
}

static int32_t launch_scores(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                             const idx_kcache& cache, const idx_rows& rows, float* scores, int64_t ld,
                             bool write_pad, hipStream_t s) {
  if (q_dtype == IDX_BF16)
    return launched(dsa::launch_score_decode(static_cast<const uint16_t*>(q), w, to_kc(cache),
                                             to_rows(rows), scores, ld, write_pad, s),
                    "indexer_score");
  return launched(dsa::launch_score_prefill(static_cast<const uint8_t*>(q), q_scale, w, to_kc(cache),
                                            to_rows(rows), scores, ld, write_pad, s),
                  "indexer_score");
}

IDX_API int32_t indexer_score(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                      int32_t heads, idx_kcache cache, idx_rows rows, float* scores, int64_t ld,
                      void* hip_stream) {
  g_err.clear();
  if (int32_t e = check_score_args(q, q_dtype, q_scale, w, heads, cache, rows)) return e;
  if (rows.rows == 0 || rows.max_row_len == 0) return IDX_OK;
  if (!scores) return fail(IDX_EINVAL, "scores must be non-NULL");
  if (!aligned(scores, 4)) return fail(IDX_EINVAL, "scores must be 4-byte aligned");
  if (ld < rows.max_row_len) return fail(IDX_EINVAL, "ld %lld < max_row_len %d", (long long)ld, rows.max_row_len);
  return launch_scores(q, q_dtype, q_scale, w, cache, rows, scores, ld, true,
                       static_cast<hipStream_t>(hip_stream));
}

static int32_t check_topk_common(int32_t rows, int32_t max_row_len, int32_t k, int32_t* out_idx) {
  if (k < 1 || k > kMaxK) return fail(IDX_EINVAL, "k=%d out of [1, %d]", k, kMaxK);
  if (rows < 0 || rows > kMaxRows) return fail(IDX_EINVAL, "rows %d out of [0, %d]", rows, kMaxRows);
  if (max_row_len < 0) return fail(IDX_EINVAL, "max_row_len must be >= 0");
  if (rows > 0 && !out_idx) return fail(IDX_EINVAL, "out_idx must be non-NULL");
  if (out_idx && !aligned(out_idx, 4)) return fail(IDX_EINVAL, "out_idx must be 4-byte aligned");
  return IDX_OK;
}

IDX_API int32_t indexer_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t rows,
                     int32_t max_row_len, int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes,
                     void* hip_stream) {
  g_err.clear();
  if (int32_t e = check_topk_common(rows, max_row_len, k, out_idx)) return e;
  if (rows == 0) return IDX_OK;
  if (!row_len) return fail(IDX_EINVAL, "row_len must be non-NULL");
  if (max_row_len > 0 && !scores) return fail(IDX_EINVAL, "scores must be non-NULL");
  if (ld < max_row_len) return fail(IDX_EINVAL, "ld %lld < max_row_len %d", (long long)ld, max_row_len);
  const size_t need = dsa::topk_ws_bytes(rows, max_row_len, k);
  if (need && (!ws || ws_bytes < need))
    return fail(IDX_EWORKSPACE, "workspace of %zu bytes required, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (need && !aligned(ws, 256)) return fail(IDX_EINVAL, "ws must be 256-byte aligned");
  return launched(dsa::launch_topk(scores, ld, row_len, rows, max_row_len, k, out_idx, nullptr,
                                   dsa::SlotMap{}, ws, static_cast<hipStream_t>(hip_stream)),
                  "indexer_topk");
}

static int32_t check_score_topk_args(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                                     int32_t heads, const idx_kcache& cache, const idx_rows& rows, int32_t k,
                                     int32_t* out_idx, int64_t* out_slots, float* out_scores) {
  if (int32_t e = check_score_args(q, q_dtype, q_scale, w, heads, cache, rows)) return e;
  if (int32_t e = check_topk_common(rows.rows, rows.max_row_len, k, out_idx)) return e;
  if (out_slots && !aligned(out_slots, 8)) return fail(IDX_EINVAL, "out_slots must be 8-byte aligned");
  if (out_scores && !aligned(out_scores, 4)) return fail(IDX_EINVAL, "out_scores must be 4-byte aligned");
  return IDX_OK;
}

static size_t score_topk_ws_bytes(int32_t rows, int32_t max_row_len, int32_t k) {
  return score_bytes(rows, max_row_len) + dsa::topk_ws_bytes(rows, max_row_len, k);
}

// The score rows go to the start of ws, the top-k lists after them.
static int32_t run_score_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                              const idx_kcache& cache, const idx_rows& rows, int32_t k, int32_t* out_idx,
                              int64_t* out_slots, float* out_scores, void* ws, hipStream_t s, const char* who) {
  float* sc = static_cast<float*>(ws);
  const int64_t ld = score_ld(rows.max_row_len);
  if (rows.max_row_len > 0)
    if (int32_t e = launch_scores(q, q_dtype, q_scale, w, cache, rows, sc, ld, false, s)) return e;
  void* tws = static_cast<uint8_t*>(ws) + score_bytes(rows.rows, rows.max_row_len);
  return launched(dsa::launch_topk(sc, ld, rows.row_len, rows.rows, rows.max_row_len, k, out_idx,
                                   out_scores, to_map(cache, rows, out_slots, k), tws, s),
                  who);
}

IDX_API int32_t indexer_score_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                           int32_t heads, idx_kcache cache, idx_rows rows, int32_t k, int32_t* out_idx,
                           int64_t* out_slots, float* out_scores, void* ws, size_t ws_bytes,
                           void* hip_stream) {
  g_err.clear();
  if (int32_t e = check_score_topk_args(q, q_dtype, q_scale, w, heads, cache, rows, k, out_idx, out_slots,
                                        out_scores))
    return e;
  if (rows.rows == 0) return IDX_OK;
  const size_t need = score_topk_ws_bytes(rows.rows, rows.max_row_len, k);
  if (!ws || ws_bytes < need)
    return fail(IDX_EWORKSPACE, "workspace of %zu bytes required, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (!aligned(ws, 256)) return fail(IDX_EINVAL, "ws must be 256-byte aligned");
  return run_score_topk(q, q_dtype, q_scale, w, cache, rows, k, out_idx, out_slots, out_scores, ws,
                        static_cast<hipStream_t>(hip_stream), "indexer_score_topk");
}

IDX_API int32_t indexer_score_topk_static(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                                          int32_t heads, idx_kcache cache, idx_rows rows, int32_t k,
                                          int32_t* out_idx, int64_t* out_slots, float* out_scores,
                                          void* hip_stream) {
  g_err.clear();
  if (int32_t e = check_score_topk_args(q, q_dtype, q_scale, w, heads, cache, rows, k, out_idx, out_slots,
                                        out_scores))
    return e;
  if (rows.rows == 0) return IDX_OK;
  const size_t need = score_topk_ws_bytes(rows.rows, rows.max_row_len, k);
  if (need > (size_t)IDX_STATIC_SCRATCH_BYTES)
    return fail(IDX_EWORKSPACE, "needs %zu bytes of scratch; the static scratch holds %zu (use indexer_score_topk "
                "with a workspace)", need, (size_t)IDX_STATIC_SCRATCH_BYTES);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* ws = nullptr;
  if (int32_t e = scratch_of_stream(s, &ws)) return e;
  return run_score_topk(q, q_dtype, q_scale, w, cache, rows, k, out_idx, out_slots, out_scores, ws, s,
                        "indexer_score_topk_static");
}

IDX_API size_t indexer_attention_workspace_bytes(int32_t rows, int32_t k, int32_t heads) {
  if (rows < 0 || rows > kMaxRows || k < 0 || k > kMaxAttnK) return 0;
  if (heads != 16 && heads != 32 && heads != 64 && heads != 128) return 0;
  return dsa::attention_ws_bytes(rows, k, heads);
}

IDX_API int32_t indexer_sparse_attention(const void* q, int32_t heads, const void* kv, int64_t num_slots,
                                         const int64_t* slots, int64_t ld_slots, int32_t k, int32_t rows,
                                         float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                         void* hip_stream) {
  g_err.clear();
  if (heads != 16 && heads != 32 && heads != 64 && heads != 128)
    return fail(IDX_EUNSUPPORTED, "heads=%d unsupported (16, 32, 64 or 128)", heads);
  if (rows < 0 || rows > kMaxRows) return fail(IDX_EINVAL, "rows %d out of [0, %d]", rows, kMaxRows);
  if (k < 0 || k > kMaxAttnK) return fail(IDX_EINVAL, "k=%d out of [0, %d]", k, kMaxAttnK);
  if (ld_slots < k) return fail(IDX_EINVAL, "ld_slots %lld < k %d", (long long)ld_slots, k);
  if (num_slots < 1 || num_slots > (int64_t)INT32_MAX) return fail(IDX_EINVAL, "num_slots must be in [1, INT32_MAX]");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(IDX_EINVAL, "scale must be finite and > 0");
  if (rows == 0) return IDX_OK;
  if (!q || !kv || !out || (k > 0 && !slots)) return fail(IDX_EINVAL, "q, kv, slots and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(IDX_EINVAL, "q, kv and out must be 16-byte aligned");
  if (slots && !aligned(slots, 8)) return fail(IDX_EINVAL, "slots must be 8-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(IDX_EINVAL, "lse must be 4-byte aligned");
  const size_t need = dsa::attention_ws_bytes(rows, k, heads);
  if (need && (!ws || ws_bytes < need))
    return fail(IDX_EWORKSPACE, "workspace of %zu bytes required, %zu given", need, ws ? ws_bytes : (size_t)0);
  if (need && !aligned(ws, 256)) return fail(IDX_EINVAL, "ws must be 256-byte aligned");
  return launched(dsa::launch_attention(static_cast<const uint16_t*>(q), heads, static_cast<const uint8_t*>(kv),
                                        num_slots, slots, ld_slots, k, rows, scale, out, lse, ws,
                                        static_cast<hipStream_t>(hip_stream)),
                  "indexer_sparse_attention");
}

IDX_API int32_t indexer_translate(const int32_t* idx, int64_t ld_idx, int32_t k, idx_kcache cache,
                                  idx_rows rows, int64_t* slots, int64_t ld_slots, void* hip_stream) {
  g_err.clear();
  if (k < 0) return fail(IDX_EINVAL, "k must be >= 0");
  if (ld_idx < k || ld_slots < k) return fail(IDX_EINVAL, "ld_idx and ld_slots must be >= k");
  if (cache.block_size != 32 && cache.block_size != 64)
    return fail(IDX_EUNSUPPORTED, "cache.block_size %d unsupported (32 or 64)", cache.block_size);
  if (cache.num_blocks < 1 || cache.num_blocks > (int64_t)INT32_MAX)
    return fail(IDX_EINVAL, "cache.num_blocks must be in [1, INT32_MAX]");
  if (int32_t e = check_rows(rows)) return e;
  if ((int64_t)rows.max_row_len > (int64_t)rows.max_blocks * cache.block_size)
    return fail(IDX_EINVAL, "max_row_len %d exceeds max_blocks*block_size", rows.max_row_len);
  if (rows.rows == 0 || k == 0) return IDX_OK;
  if (!idx || !slots) return fail(IDX_EINVAL, "idx and slots must be non-NULL");
  if (!aligned(idx, 4)) return fail(IDX_EINVAL, "idx must be 4-byte aligned");
  if (!aligned(slots, 8)) return fail(IDX_EINVAL, "slots must be 8-byte aligned");
  return launched(dsa::launch_translate(idx, ld_idx, rows.rows, k, to_map(cache, rows, slots, ld_slots),
                                        static_cast<hipStream_t>(hip_stream)),
                  "indexer_translate");
}

}  // extern "C"
