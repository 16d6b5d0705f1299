"""Every entry point with nothing to do (zero vectors, rows or slots) returns success
through the binding, launches nothing that writes, and leaves its outputs untouched."""
import pytest
import torch

import sparse_attention_token_store_amd as dsa

from _hip import i32, note

pytestmark = pytest.mark.gpu


def empty(*shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def test_empty_calls():
    note("zero-size calls of every entry point")
    buf = torch.full((dsa.cache_bytes(dsa.IDX_FP8_E4M3, 64, 4),), 0x5A, dtype=torch.uint8, device="cuda")
    cache = dsa.kcache(buf, dsa.IDX_FP8_E4M3, 64, 4)
    before = buf.clone()
    # store and query preparation of zero vectors
    dsa.index_k_store(empty(0, 128, dtype=torch.bfloat16), empty(0, dtype=torch.int32), empty(0, dtype=torch.int64),
                      cache, dsa.IDX_STORE_ALL)
    dsa.indexer_q_prep(empty(0, 64, 128, dtype=torch.bfloat16), empty(0, dtype=torch.int32), dsa.IDX_STORE_ALL,
                       out_bf16=empty(0, 64, 128, dtype=torch.bfloat16))
    dsa.indexer_quant_fp8(empty(0, 128, dtype=torch.bfloat16), empty(0, 128, dtype=torch.uint8),
                          empty(0, dtype=torch.float32))
    # scoring and selection over zero rows
    bt, rs, rl = i32([[0, 1, 2, 3]]), empty(0, dtype=torch.int32), empty(0, dtype=torch.int32)
    rows0 = dsa.rows_desc(bt, rs, rl, 256)
    q = empty(0, 64, 128, dtype=torch.bfloat16)
    w = empty(0, 64, dtype=torch.float32)
    dsa.indexer_score(q, w, cache, rows0, empty(0, 256, dtype=torch.float32))
    dsa.indexer_topk(empty(0, 256, dtype=torch.float32), rl, 256, 512, empty(0, 512, dtype=torch.int32))
    dsa.indexer_score_topk(q, w, cache, rows0, 512, empty(0, 512, dtype=torch.int32), None,
                           out_scores=empty(0, 512, dtype=torch.float32), out_slots=empty(0, 512, dtype=torch.int64))
    dsa.indexer_score_topk_static(q, w, cache, rows0, 512, empty(0, 512, dtype=torch.int32))
    dsa.indexer_translate(empty(0, 512, dtype=torch.int32), cache, rows0, empty(0, 512, dtype=torch.int64))
    # attention over zero rows, and rows with k = 0
    kv = torch.zeros((8, 512), dtype=torch.bfloat16, device="cuda")
    assert dsa.alloc_attention_workspace(0, 512, 16) is None
    dsa.indexer_sparse_attention(empty(0, 16, 512, dtype=torch.bfloat16), kv, empty(0, 512, dtype=torch.int64),
                                 empty(0, 16, 512, dtype=torch.float32))
    out = torch.full((2, 16, 512), 7.0, device="cuda")
    lse = torch.full((2, 16), 7.0, device="cuda")
    dsa.indexer_sparse_attention(torch.zeros((2, 16, 512), dtype=torch.bfloat16, device="cuda"), kv,
                                 empty(2, 0, dtype=torch.int64), out, k=0, lse=lse)
    # a selection of 0 entries is a decided result: zero output and lse = -inf
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    assert bool((out == 0).all()) and bool(torch.isneginf(lse).all())
