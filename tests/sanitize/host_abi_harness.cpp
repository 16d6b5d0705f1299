// Host-only exercise of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizers.py builds it with the library's host code instrumented):
// every workspace-size query over extreme and random arguments, and a refused call of
// each kind of entry point.  Nothing is launched, so it needs no GPU.
#include <cstdio>
#include <cstdint>
#include <random>
#include "dsa_indexer.h"
int main() {
  std::mt19937_64 g(1);
  const int32_t vals[] = {-2147483647 - 1, -65536, -1, 0, 1, 2, 3, 4, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128,
                          511, 512, 513, 1023, 1024, 1025, 2047, 2048, 4096, 8191, 8192, 8193, 16384, 32767,
                          32768, 36864, 36865, 65535, 65536, 65537, 1 << 20, (1 << 30), 2147483647};
  size_t acc = 0; long n = 0;
  for (int op : {0, 1, 2, 3})
    for (int32_t r : vals) for (int32_t L : vals) for (int32_t k : vals) { acc += indexer_workspace_bytes(op, r, L, k); ++n; }
  for (int32_t r : vals) for (int32_t k : vals) for (int32_t h : {-16, 0, 8, 16, 24, 32, 48, 64, 96, 128, 256})
    { acc += indexer_attention_workspace_bytes(r, k, h); ++n; }
  std::uniform_int_distribution<int64_t> any(INT32_MIN, INT32_MAX);
  for (int i = 0; i < 200000; ++i) {
    acc += indexer_workspace_bytes(1 + (int)(g() % 2), (int32_t)any(g), (int32_t)any(g), (int32_t)any(g));
    acc += indexer_attention_workspace_bytes((int32_t)any(g), (int32_t)any(g), (int32_t)any(g));
    n += 2;
  }
  // refused calls: every one fails validation before any HIP call
  void* fake = (void*)(uintptr_t)(1 << 20);
  idx_kcache c{fake, 2, 64, 10};
  idx_rows rows{(const int32_t*)fake, 4, 2, (const int32_t*)fake, (const int32_t*)fake, 4, 100};
  int bad = 0;
  bad += indexer_topk((const float*)fake, 100, (const int32_t*)fake, 4, 100, 0, (int32_t*)fake, nullptr, 0, nullptr) == IDX_EINVAL;
  bad += indexer_score(fake, 7, nullptr, (const float*)fake, 64, c, rows, (float*)fake, 128, nullptr) == IDX_EINVAL;
  bad += indexer_sparse_attention(fake, 24, fake, 10, (const int64_t*)fake, 4, 4, 2, 1.0f, (float*)fake, nullptr, nullptr, 0, nullptr) == IDX_EUNSUPPORTED;
  bad += index_k_store(fake, -1, nullptr, (const int64_t*)fake, c, 0, 1e-6f, 1e4f, 64, nullptr, nullptr) == IDX_EINVAL;
  bad += indexer_q_prep(fake, 7, 4, nullptr, 0, 1e-6f, 1e4f, 64, fake, nullptr, nullptr, nullptr, nullptr) == IDX_EINVAL;
  std::printf("queries %ld (sum %zu), refused calls ok %d/5, last error: %s\n", n, acc, bad, indexer_last_error());
  return bad == 5 ? 0 : 1;
}
