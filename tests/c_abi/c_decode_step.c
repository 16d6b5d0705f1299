/*
 * A plain C caller of the indexer library: only include/dsa_indexer.h and the HIP
 * runtime API, no Python and no torch.  It stores the index keys of two sequences
 * into a paged fp8 cache through a shuffled block table, runs the fused score +
 * top-k for three query rows (two of them on the same sequence), checks that a
 * refused call reports its error, and writes every input and output to a file that
 * the test compares with the oracle.
 *
 *   usage: c_decode_step OUT_FILE
 *
 * File layout (little-endian): int32 magic 0x43414249 ("CABI"), then int32 nseq,
 * rows, heads, k, bs, num_blocks, max_blocks, max_row_len, then seq_len[nseq],
 * block_table[nseq][max_blocks], row_seq[rows], row_len[rows] (int32), keys of every
 * sequence in order (bf16 bits [sum seq_len][128]), q (bf16 bits [rows][heads][128]),
 * w (fp32 [rows][heads]), out_idx (int32 [rows][k]), out_scores (fp32 [rows][k]).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dsa_indexer.h"

enum { NSEQ = 2, ROWS = 3, HEADS = 64, DIM = 128, K = 256, BS = 64 };
static const int kSeqLen[NSEQ] = {700, 1300};
static const int kRowSeq[ROWS] = {0, 1, 1};
static const int kRowLen[ROWS] = {700, 1300, 900};

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

#define IDX_OK_OR_DIE(call)                                                   \
  do {                                                                        \
    int32_t s_ = (call);                                                      \
    if (s_ != IDX_OK) {                                                       \
      fprintf(stderr, "%s returned %d: %s\n", #call, s_, indexer_last_error()); \
      exit(3);                                                                \
    }                                                                         \
  } while (0)

/* 32-bit linear congruential generator (Numerical Recipes constants) */
static uint32_t g_state = 12345u;
static float uniform(void) { /* in [-1, 1) */
  g_state = g_state * 1664525u + 1013904223u;
  return (float)(g_state >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void* dev_copy(const void* host, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes));
  HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUT_FILE\n", argv[0]);
    return 1;
  }
  if (indexer_abi_version() != IDX_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", indexer_abi_version(), IDX_ABI_VERSION);
    return 4;
  }

  /* block tables: sequence b's logical block j lives in physical block
   * (7 * global_index + 3) mod num_blocks, a permutation of the pool */
  int max_blocks = 0, num_blocks = 0, total = 0;
  for (int b = 0; b < NSEQ; ++b) {
    const int nb = (kSeqLen[b] + BS - 1) / BS;
    if (nb > max_blocks) max_blocks = nb;
    num_blocks += nb;
    total += kSeqLen[b];
  }
  int32_t* table = calloc((size_t)NSEQ * max_blocks, sizeof(int32_t));
  for (int b = 0, g = 0; b < NSEQ; ++b) {
    const int nb = (kSeqLen[b] + BS - 1) / BS;
    for (int j = 0; j < max_blocks; ++j) table[b * max_blocks + j] = j < nb ? (7 * g++ + 3) % num_blocks : -1;
  }

  /* keys of both sequences, their store slots, the queries and the weights */
  uint16_t* keys = malloc((size_t)total * DIM * 2);
  int64_t* slots = malloc((size_t)total * 8);
  for (int b = 0, t = 0; b < NSEQ; ++b)
    for (int p = 0; p < kSeqLen[b]; ++p, ++t) {
      for (int d = 0; d < DIM; ++d) keys[(size_t)t * DIM + d] = to_bf16(uniform());
      slots[t] = (int64_t)table[b * max_blocks + p / BS] * BS + p % BS;
    }
  uint16_t* q = malloc((size_t)ROWS * HEADS * DIM * 2);
  for (size_t i = 0; i < (size_t)ROWS * HEADS * DIM; ++i) q[i] = to_bf16(uniform());
  float* w = malloc((size_t)ROWS * HEADS * 4);
  for (int i = 0; i < ROWS * HEADS; ++i) w[i] = (uniform() + 1.0f) / 16.0f;

  /* device buffers, all owned by this program */
  const size_t cache_bytes = (size_t)num_blocks * BS * 132;
  void* cache_base = NULL;
  HIP_OK(hipMalloc(&cache_base, cache_bytes));
  HIP_OK(hipMemset(cache_base, 0xFF, cache_bytes));
  void* d_keys = dev_copy(keys, (size_t)total * DIM * 2);
  void* d_slots = dev_copy(slots, (size_t)total * 8);
  void* d_q = dev_copy(q, (size_t)ROWS * HEADS * DIM * 2);
  void* d_w = dev_copy(w, (size_t)ROWS * HEADS * 4);
  void* d_table = dev_copy(table, (size_t)NSEQ * max_blocks * 4);
  void* d_seq = dev_copy(kRowSeq, sizeof kRowSeq);
  void* d_len = dev_copy(kRowLen, sizeof kRowLen);
  int32_t* d_idx = NULL;
  float* d_sc = NULL;
  HIP_OK(hipMalloc((void**)&d_idx, (size_t)ROWS * K * 4));
  HIP_OK(hipMalloc((void**)&d_sc, (size_t)ROWS * K * 4));

  idx_kcache cache = {cache_base, IDX_FP8_E4M3, BS, num_blocks};
  int max_row_len = 0;
  for (int r = 0; r < ROWS; ++r)
    if (kRowLen[r] > max_row_len) max_row_len = kRowLen[r];
  idx_rows rows = {(const int32_t*)d_table, max_blocks, NSEQ, (const int32_t*)d_seq, (const int32_t*)d_len,
                   ROWS, max_row_len};

  const size_t ws_bytes = indexer_workspace_bytes(IDX_OP_SCORE_TOPK, ROWS, max_row_len, K);
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes));

  /* fp8 store of the keys as given (flags 0), then the fused selection */
  IDX_OK_OR_DIE(index_k_store(d_keys, total, NULL, (const int64_t*)d_slots, cache, 0u, 1e-6f, 10000.0f, 64,
                              NULL, NULL));
  IDX_OK_OR_DIE(indexer_score_topk(d_q, IDX_BF16, NULL, (const float*)d_w, HEADS, cache, rows, K, d_idx, NULL,
                                   d_sc, ws, ws_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());

  /* a refused call: k = 0 is out of range, reported before anything is launched */
  if (indexer_topk(NULL, max_row_len, (const int32_t*)d_len, ROWS, max_row_len, 0, d_idx, NULL, 0, NULL) !=
          IDX_EINVAL ||
      strstr(indexer_last_error(), "k=0") == NULL) {
    fprintf(stderr, "k = 0 was not refused as expected: %s\n", indexer_last_error());
    return 5;
  }

  int32_t* idx = malloc((size_t)ROWS * K * 4);
  float* sc = malloc((size_t)ROWS * K * 4);
  HIP_OK(hipMemcpy(idx, d_idx, (size_t)ROWS * K * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(sc, d_sc, (size_t)ROWS * K * 4, hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) {
    perror(argv[1]);
    return 6;
  }
  const int32_t head[9] = {0x43414249, NSEQ, ROWS, HEADS, K, BS, num_blocks, max_blocks, max_row_len};
  fwrite(head, 4, 9, f);
  fwrite(kSeqLen, 4, NSEQ, f);
  fwrite(table, 4, (size_t)NSEQ * max_blocks, f);
  fwrite(kRowSeq, 4, ROWS, f);
  fwrite(kRowLen, 4, ROWS, f);
  fwrite(keys, 2, (size_t)total * DIM, f);
  fwrite(q, 2, (size_t)ROWS * HEADS * DIM, f);
  fwrite(w, 4, (size_t)ROWS * HEADS, f);
  fwrite(idx, 4, (size_t)ROWS * K, f);
  fwrite(sc, 4, (size_t)ROWS * K, f);
  fclose(f);

  HIP_OK(hipFree(cache_base));
  HIP_OK(hipFree(d_keys));
  HIP_OK(hipFree(d_slots));
  HIP_OK(hipFree(d_q));
  HIP_OK(hipFree(d_w));
  HIP_OK(hipFree(d_table));
  HIP_OK(hipFree(d_seq));
  HIP_OK(hipFree(d_len));
  HIP_OK(hipFree(d_idx));
  HIP_OK(hipFree(d_sc));
  HIP_OK(hipFree(ws));
  free(table);
  free(keys);
  free(slots);
  free(q);
  free(w);
  free(idx);
  free(sc);
  printf("c_decode_step: %d rows, %d keys, k = %d, written to %s\n", ROWS, total, K, argv[1]);
  return 0;
}
