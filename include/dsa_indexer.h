/*
 * dsa_indexer.h - C ABI of the DeepSeek sparse-attention (DSA) lightning-indexer hot
 * path on AMD Instinct MI355X (gfx950): index-K store, per-key relevance score and
 * causal top-k over a paged index-K cache.
 *
 * Sources (web pages, cited by title and section):
 *   [ATOM-1507]  "[DeepSeek-V4] index_topk=1024 sparse indexer can't recall verbatim
 *                lines from ~18k+ prompts" (ROCm/ATOM issue 1507)
 *   [PIVOT-EDIT] "The Pivot: A Single Edit That Finally Fixed DeepSeek V4's
 *                Long-Context Recall Failure"
 *   [HYPOTHESIS] "The Hypothesis That Refused to Die: When Synthetic Tests
 *                Contradict Real-World Failure"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as device buffers are device pointers owned by the caller.  The
 *    library never allocates or frees device memory, never synchronises a stream and
 *    never reads device data on the host.  Scratch space is the caller's `ws`
 *    (indexer_score_topk_static alone uses a static array of the library instead).
 *  - All work is queued on `hip_stream` (a hipStream_t; NULL = the null stream) and
 *    is asynchronous.  No call records a memset, so calls can be captured in a HIP
 *    graph.
 *  - Errors: argument checks run on the host before anything is launched; on failure
 *    the call returns IDX_EINVAL / IDX_EUNSUPPORTED / IDX_EWORKSPACE, launches
 *    nothing and sets a message readable with indexer_last_error() (thread-local).
 *    A failed launch returns IDX_ELAUNCH.  Nothing throws across the ABI.
 *  - Device-resident indices (block ids, slots, positions, row lengths, row
 *    sequences) cannot be checked on the host.  The kernels never access memory out
 *    of bounds because of them: a block id outside [0, num_blocks) scores NaN, a
 *    store slot outside the pool is skipped, row_len is clamped to
 *    [0, max_row_len] and a row_seq outside [0, num_seqs) scores NaN.
 *  - head_dim is 128 throughout.  Outputs are bit-deterministic: there are no
 *    floating-point atomics.
 *  - Calls are re-entrant; the only global state is the thread-local error string
 *    and the static scratch array of indexer_score_topk_static (one per GPU).
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IDX_ABI_VERSION 2
#define IDX_HEAD_DIM 128

typedef enum {
  IDX_OK = 0,
  IDX_EINVAL = -1,        /* bad argument (null pointer, size, alignment, range) */
  IDX_EUNSUPPORTED = -2,  /* valid but unsupported combination (dtype pair, heads) */
  IDX_ELAUNCH = -3,       /* kernel launch failed (HIP error) */
  IDX_EWORKSPACE = -4     /* workspace missing or smaller than required */
} idx_status;

typedef enum { IDX_BF16 = 1, IDX_FP8_E4M3 = 2, IDX_MXFP4 = 3 } idx_dtype;

/* index_k_store flags: which steps precede the quantise-and-scatter.  flags = 0
 * stores the input as given (quantised for an fp8 cache). */
enum { IDX_STORE_RMSNORM = 1u, IDX_STORE_ROPE = 2u, IDX_STORE_HADAMARD = 4u };

/* ops for indexer_workspace_bytes */
enum { IDX_OP_TOPK = 1, IDX_OP_SCORE_TOPK = 2 };

/*
 * Paged index-K cache ([ATOM-1507] "How it was isolated": paged index-K cache read
 * through a block table at block size 32 or 64; [PIVOT-EDIT] "Assumptions and Input
 * Knowledge": 132 bytes per token for fp8, 256 for bf16).
 *   base        device pointer to block 0, 256-byte aligned.
 *   dtype       IDX_BF16: block b holds block_size rows of 128 bf16 (256 B each),
 *                 at base + b*block_size*256.
 *               IDX_FP8_E4M3: block b is block_size*132 bytes at
 *                 base + b*block_size*132: first block_size*128 bytes of OCP e4m3fn
 *                 codes (row-major, 128 per token), then block_size fp32 scales.
 *                 Token value = scale * decode(code).
 *               IDX_MXFP4 (the fp4 index keys of [ATOM-1507] "Where",
 *                 fp4_act_quant_inplace(kv, 32), read as OCP MXFP4): block b is
 *                 block_size*68 bytes at base + b*block_size*68: first
 *                 block_size*64 bytes of e2m1 codes (64 per token; element 2i in
 *                 the low nibble of byte i), then block_size*4 e8m0 bytes (the
 *                 scale 2^(E-127) of token elements 32j .. 32j+31 is byte 4t+j).
 *                 Scored with bf16 queries (widened exactly to bf16) or fp8
 *                 queries (the e8m0 bytes are the scaled MFMA's block scales).
 *   block_size  tokens per block: 32 or 64.
 *   num_blocks  blocks in the pool (physical block ids are in [0, num_blocks)).
 */
typedef struct {
  void* base;
  int32_t dtype;
  int32_t block_size;
  int64_t num_blocks;
} idx_kcache;

/*
 * Query rows and what each row may see (causal / committed-key mask, [ATOM-1507]
 * "Analysis / question" and "How it was isolated").
 *   block_table  device int32 [num_seqs][max_blocks]: physical block of each
 *                logical block of each sequence.
 *   row_seq      device int32 [rows]: the sequence a query row reads.
 *   row_len      device int32 [rows]: row r sees key positions 0..row_len[r]-1
 *                (its own key included, stored before scoring).
 *   max_row_len  host-known upper bound of every row_len (sizes the grid and the
 *                score rows); must be <= max_blocks*block_size.
 */
typedef struct {
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t num_seqs;
  const int32_t* row_seq;
  const int32_t* row_len;
  int32_t rows;
  int32_t max_row_len;
} idx_rows;

/*
 * index_k_store - write n index keys into the paged cache.
 * Steps ([PIVOT-EDIT] "The Reasoning Behind the Edit": the unfused key path
 * normalises, applies RoPE and rotates before it writes the cache; [ATOM-1507]
 * "Root cause found"/"Where": interleaved RoPE on the trailing rope_dim, then the
 * Walsh-Hadamard rotation that must match the query's; the store is the analog of
 * the pages' indexer_k_quant_and_cache / fused compressor store), each enabled by a
 * flag:
 *   RMSNorm   y = x / sqrt(mean(x^2) + rms_eps), unit gain
 *   RoPE      pair i = (y[o+2i], y[o+2i+1]), o = 128 - rope_dim, rotated by
 *             pos * rope_base^(-2i/rope_dim) (angle formed in double precision)
 *   Hadamard  y = H y / sqrt(128), H the 128x128 Sylvester-order Walsh matrix
 *   store     fp8 cache: amax = max|y|, s = amax/448 (correctly rounded fp32
 *             division; s = 1 when amax < 2^-100), code = e4m3(y/s) rounded to
 *             nearest even with saturation; bf16 cache: y rounded to nearest even;
 *             MXFP4 cache: per 32-element block, e = floor(log2(amax)) - 2 within
 *             [-127, 127] (0 for an all-zero block), codes = e2m1(y * 2^-e) to the
 *             nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even mantissa bit,
 *             saturating at 6), e8m0 byte e + 127.
 * Arguments:
 *   x_bf16        device bf16 [n][128] hidden rows (row-major).
 *   n             number of tokens (0 is a no-op).
 *   positions     device int32 [n]: RoPE positions (read only with IDX_STORE_ROPE;
 *                 may be NULL otherwise).
 *   slot_mapping  device int64 [n]: destination slot = block*block_size + offset;
 *                 a negative slot skips the token.
 *   prequant_dbg  NULL, or device fp32 [n][128] receiving the rows just before
 *                 quantisation / rounding (debug output).
 *   rope_dim      even, 2..128 (read only with IDX_STORE_ROPE).
 */
int32_t index_k_store(const void* x_bf16, int64_t n, const int32_t* positions,
                      const int64_t* slot_mapping, idx_kcache cache, uint32_t flags,
                      float rms_eps, float rope_base, int32_t rope_dim, float* prequant_dbg,
                      void* hip_stream);

/*
 * indexer_q_prep - prepare index queries with the index key's chain.
 * [ATOM-1507] "Where": the index query goes through interleaved RoPE on the trailing
 * rope_dim, then a Hadamard rotation, then fp8 quantisation; "Root cause found":
 * the key must carry the same rotation, because (H q).(H k) = q.k for the
 * orthogonal H while (H q).k is a scrambled product ("Recommended fix" (A) drops
 * the query's rotation instead: call this without IDX_STORE_HADAMARD).
 * Every (row, head) vector goes through the steps of index_k_store selected by
 * flags (RMSNorm, RoPE, Hadamard, same definitions), all heads of row r at
 * position positions[r]; then
 *   out_bf16          y rounded to bf16 (nearest even), and/or
 *   codes / scales    the per-vector fp8 quantisation of indexer_quant_fp8.
 * Arguments:
 *   q_bf16        device bf16 [n_vec][128] = [rows][heads][128], row-major.
 *   n_vec         rows * heads (0 is a no-op); must be a multiple of heads, with
 *                 rows * ceil(heads / 4) <= 4 * INT32_MAX.
 *   positions     device int32 [rows] (read only with IDX_STORE_ROPE).
 *   out_bf16      NULL or device bf16 [n_vec][128].
 *   codes, scales both NULL, or device uint8 [n_vec][128] and fp32 [n_vec].
 *   prequant_dbg  NULL or device fp32 [n_vec][128]: y before rounding/quantisation.
 * At least one output must be requested when n_vec > 0 (n_vec = 0 is a no-op, with
 * any pointers).  Errors: IDX_EINVAL for a bad size, flag, rope parameter, missing
 * pointer or misaligned pointer (q_bf16, out_bf16 and prequant_dbg 16-byte; codes
 * 8-byte; scales and positions 4-byte).
 */
int32_t indexer_q_prep(const void* q_bf16, int64_t n_vec, int32_t heads, const int32_t* positions,
                       uint32_t flags, float rms_eps, float rope_base, int32_t rope_dim, void* out_bf16,
                       uint8_t* codes, float* scales, float* prequant_dbg, void* hip_stream);

/*
 * indexer_quant_fp8 - per-vector absmax fp8 quantisation of contiguous vectors of
 * 128 values (the query-side fp8 step of the pages' rope_rotate_activation,
 * [ATOM-1507] "Where"), with exactly the same rule as the fp8 store.
 *   x_bf16  device bf16 [n_vec][128];  codes  device uint8 [n_vec][128];
 *   scales  device fp32 [n_vec].
 */
int32_t indexer_quant_fp8(const void* x_bf16, int64_t n_vec, uint8_t* codes, float* scales,
                          void* hip_stream);

/*
 * indexer_score - relevance of every visible cached key for every query row:
 *     scores[r][p] = sum_h w[r][h] * max(0, q[r][h] . k[p])      for p < row_len[r]
 *     scores[r][p] = -inf                         for row_len[r] <= p < max_row_len
 * (the lightning-indexer q.k score, [ATOM-1507] "Root cause found"; a compressed
 * query-key dot product, [HYPOTHESIS] "The Context"; per-head weights and a
 * positive softmax scale, [HYPOTHESIS] "The Bash Command", folded into w).  An fp8
 * key contributes scale_p * (q . decode(codes_p)); the per-key scale is applied
 * after the head sum.  An fp8 query contributes q_scale[r][h] * decode(code).
 * Zero scores are +0.
 *   q        device [rows][heads][128]: bf16 (q_dtype IDX_BF16) or e4m3 codes
 *            (IDX_FP8_E4M3, from indexer_quant_fp8).
 *   q_scale  device fp32 [rows][heads] for fp8 q, else ignored (may be NULL).
 *   w        device fp32 [rows][heads].
 *   heads    64 (v1).
 *   scores   device fp32 [rows][ld], ld >= max_row_len; columns >= max_row_len are
 *            not written.
 * Supported (q, key) dtypes: (bf16, bf16), (bf16, fp8), (bf16, MXFP4), (fp8, fp8),
 * (fp8, MXFP4).  (fp8, bf16) returns IDX_EUNSUPPORTED.  A key whose block id lies
 * outside [0, num_blocks) scores NaN; only that block's keys are affected.
 */
int32_t indexer_score(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                      int32_t heads, idx_kcache cache, idx_rows rows, float* scores, int64_t ld,
                      void* hip_stream);

/*
 * indexer_topk - causal top-k of score rows ([ATOM-1507] "Summary": index_topk 512
 * or 1024; "How it was isolated": the per-row top-k is judged against torch.topk).
 * Row r selects, among positions p < row_len[r], the k largest scores, ties broken
 * by the lower position (+0 and -0 are equal).  out_idx[r] holds the selected
 * positions in ascending order followed by -1 padding when row_len[r] < k.
 * A NaN score, of either sign and any payload, ranks above every number, and NaNs
 * tie among themselves (torch.topk's order): a key of a bad block id, which scores
 * NaN, is selected first.
 *   scores   device fp32 [rows][ld];  row_len  device int32 [rows].
 *   k        1..8192.
 *   out_idx  device int32 [rows][k].
 *   ws       device workspace of at least
 *            indexer_workspace_bytes(IDX_OP_TOPK, rows, max_row_len, k) bytes,
 *            256-byte aligned (NULL allowed when that size is 0).
 */
int32_t indexer_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t rows,
                     int32_t max_row_len, int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes,
                     void* hip_stream);

/*
 * indexer_score_topk - indexer_score followed by indexer_topk in one call (the
 * pages' prefill orchestration and the decode selection, [ATOM-1507] "Recommended
 * fix" and "How it was isolated").  Same arguments as the two calls; the scores
 * live in the workspace.
 *   out_idx     device int32 [rows][k] (as indexer_topk).
 *   out_slots   NULL, or device int64 [rows][k]: the physical cache slot of each
 *               selected position, as indexer_translate maps it, written by the
 *               top-k's last pass (-1 for padding).
 *   out_scores  NULL, or device fp32 [rows][k]: the score of each selected
 *               position, -inf for padding.
 *   ws          at least indexer_workspace_bytes(IDX_OP_SCORE_TOPK, rows,
 *               max_row_len, k) bytes, 256-byte aligned.
 */
int32_t indexer_score_topk(const void* q, int32_t q_dtype, const float* q_scale, const float* w,
                           int32_t heads, idx_kcache cache, idx_rows rows, int32_t k,
                           int32_t* out_idx, int64_t* out_slots, float* out_scores, void* ws,
                           size_t ws_bytes, void* hip_stream);

/*
 * indexer_score_topk_static - indexer_score_topk for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and results as indexer_score_topk, without ws:
 * the score rows and candidate lists live in a static device array of
 * IDX_STATIC_SCRATCH_BYTES per GPU, which the library holds from the first call on
 * that GPU until the process ends.  The call allocates and frees nothing.
 *   Limit: indexer_workspace_bytes(IDX_OP_SCORE_TOPK, rows, max_row_len, k) must not
 *   exceed IDX_STATIC_SCRATCH_BYTES (e.g. 32 rows of up to ~200k keys, or 4 rows of
 *   1M keys at k = 1024); larger calls return IDX_EWORKSPACE and launch nothing.
 *   Sharing: every call on one GPU uses that GPU's one array, and nothing in it needs
 *   to start at zero, but calls that overlap in time on one GPU (different streams,
 *   or host threads without ordering) race on it and must be serialised by the caller.
 */
#define IDX_STATIC_SCRATCH_BYTES (32u << 20)
int32_t indexer_score_topk_static(const void* q, int32_t q_dtype, const float* q_scale,
                                  const float* w, int32_t heads, idx_kcache cache, idx_rows rows,
                                  int32_t k, int32_t* out_idx, int64_t* out_slots,
                                  float* out_scores, void* hip_stream);

/*
 * indexer_translate - selected logical key positions -> physical cache slots (the
 * logical -> physical step after the top-k, which must be right for arbitrary index
 * lists, [ATOM-1507] "How it was isolated").  For row r < rows.rows and j < k, with
 * t = idx[r*ld_idx + j], s = rows.row_seq[r] and bs = cache.block_size:
 *   slots[r*ld_slots + j] = b*bs + t%bs,  b = rows.block_table[s*max_blocks + t/bs],
 * when 0 <= t < min(row_len[r], max_row_len), 0 <= s < num_seqs, t/bs < max_blocks
 * and 0 <= b < cache.num_blocks; otherwise -1 (so -1 padding stays -1).
 *   idx    device int32 [rows][ld_idx];  slots  device int64 [rows][ld_slots].
 *   cache  only block_size and num_blocks are read (base may be NULL).
 * Errors: IDX_EINVAL for k < 0, a stride below k, bad rows/cache geometry, missing
 * or misaligned pointers (idx 4-byte, slots 8-byte); IDX_EUNSUPPORTED for a block
 * size other than 32 or 64.  rows.rows == 0 or k == 0 is a no-op.
 */
int32_t indexer_translate(const int32_t* idx, int64_t ld_idx, int32_t k, idx_kcache cache,
                          idx_rows rows, int64_t* slots, int64_t ld_slots, void* hip_stream);

/*
 * indexer_sparse_attention - decode attention of every query head over the KV
 * states of its row's selected slots only (the consumer of the selections:
 * [ATOM-1507] "How it was isolated" checks the decode attention kernel after the
 * logical -> physical translation; "Root cause found": a key the selection drops is
 * invisible to sparse attention).  The main KV cache holds one compressed KV state
 * of head_dim 512 per token ([PIVOT-EDIT] "Assumptions and Input Knowledge"), which
 * serves as key and value for every head (multi-query latent attention, absorbed
 * form).  For row r, head h and the listed slots s_1..s_n (entries < 0 skipped):
 *     x_j = scale * q[r][h] . kv[s_j]
 *     out[r][h] = sum_j exp(x_j - m) kv[s_j] / sum_j exp(x_j - m),  m = max_j x_j
 *     lse[r][h] = log sum_j exp(x_j)          (so disjoint sets merge exactly)
 * A row that lists nothing gets out = 0 and lse = -inf; a listed slot >= num_slots
 * is never read and makes its row's out and lse NaN.  Scores and sums are fp32;
 * the probabilities meet the KV states in bf16 (MFMA) with fp32 accumulation.
 *   q          device bf16 [rows][heads][512], 16-byte aligned.
 *   heads      16, 32, 64 or 128 query heads.
 *   kv         device bf16 [num_slots][512]: slot s = block*block_size + offset of
 *              a paged cache with 512*2-byte tokens (any block size), 16-byte
 *              aligned; num_slots 1 .. INT32_MAX.
 *   slots      device int64 [rows][ld_slots], 8-byte aligned, ld_slots >= k: the
 *              first k entries of each row are its list (indexer_score_topk's
 *              out_slots or indexer_translate's); may be NULL when k = 0.
 *   k          0 .. 65536.  rows  0 .. 65535.  scale  finite, > 0 (e.g. 1/sqrt(512)).
 *   out        device fp32 [rows][heads][512], 16-byte aligned.
 *   lse        NULL or device fp32 [rows][heads].
 *   ws         indexer_attention_workspace_bytes(rows, k, heads) bytes (0: may be
 *              NULL), 256-byte aligned: per-split partial results, caller-owned,
 *              contents on entry unused.
 * Errors: IDX_EUNSUPPORTED for another head count; IDX_EINVAL for a size, stride,
 * scale, null or misaligned pointer out of the ranges above; IDX_EWORKSPACE for a
 * missing or short workspace.  The caller keeps ownership of every buffer; nothing
 * is allocated, synchronised or freed.
 */
int32_t indexer_sparse_attention(const void* q, int32_t heads, const void* kv, int64_t num_slots,
                                 const int64_t* slots, int64_t ld_slots, int32_t k, int32_t rows,
                                 float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                 void* hip_stream);

/* Workspace bytes of indexer_sparse_attention (0 when none is needed, or on bad
 * arguments). */
size_t indexer_attention_workspace_bytes(int32_t rows, int32_t k, int32_t heads);

/* Workspace bytes needed by an op (IDX_OP_TOPK or IDX_OP_SCORE_TOPK); 0 on bad
 * arguments. */
size_t indexer_workspace_bytes(int32_t op, int32_t rows, int32_t max_row_len, int32_t k);

/* Message describing the last failure on the calling thread ("" if none). */
const char* indexer_last_error(void);

/* IDX_ABI_VERSION of the built library. */
int32_t indexer_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_H */
