"""Refused calls on the GPU: with device tensors, the binding's shape checks raise
ValueError, and arguments the library refuses raise IndexerError with the library's
status and message.  Nothing is written in either case."""
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from synth import gen

from _hip import GpuWorkload, i32, note

pytestmark = pytest.mark.gpu


def dev(*shape, dtype=torch.float32, fill=7):
    return torch.full(shape, fill, dtype=dtype, device="cuda")


def test_shape_mismatches_raise_value_error():
    note("binding shape checks")
    bf, u8, i32_, i64 = torch.bfloat16, torch.uint8, torch.int32, torch.int64
    buf = dev(dsa.cache_bytes(dsa.IDX_FP8_E4M3, 64, 2), dtype=u8, fill=0)
    cache = dsa.kcache(buf, dsa.IDX_FP8_E4M3, 64, 2)
    with pytest.raises(ValueError, match="slot_mapping"):
        dsa.index_k_store(dev(4, 128, dtype=bf), None, dev(3, dtype=i64), cache)
    with pytest.raises(ValueError, match="positions"):
        dsa.indexer_q_prep(dev(4, 64, 128, dtype=bf), dev(3, dtype=i32_), dsa.IDX_STORE_ROPE,
                           out_bf16=dev(4, 64, 128, dtype=bf))
    with pytest.raises(ValueError, match="codes"):
        dsa.indexer_q_prep(dev(4, 64, 128, dtype=bf), None, 0, codes=dev(4, 64, 64, dtype=u8),
                           scales=dev(4, 64))
    with pytest.raises(ValueError, match="codes must match"):
        dsa.indexer_quant_fp8(dev(4, 128, dtype=bf), dev(4, 64, dtype=u8), dev(4))
    rows = dsa.rows_desc(i32([[0, 1]]), i32([0, 0]), i32([10, 20]), 100)
    with pytest.raises(ValueError, match="out_slots"):
        dsa.indexer_score_topk(dev(2, 64, 128, dtype=bf), dev(2, 64), cache, rows, 8, dev(2, 8, dtype=i32_),
                               None, out_slots=dev(2, 4, dtype=i64))
    with pytest.raises(ValueError, match="idx and out_slots"):
        dsa.indexer_translate(dev(2, 8, dtype=i32_), cache, rows, dev(2, 4, dtype=i64))
    with pytest.raises(ValueError, match="out"):
        dsa.indexer_sparse_attention(dev(2, 16, 512, dtype=bf), dev(8, 512, dtype=bf), dev(2, 4, dtype=i64),
                                     dev(2, 16, 256))
    with pytest.raises(ValueError, match="lse"):
        dsa.indexer_sparse_attention(dev(2, 16, 512, dtype=bf), dev(8, 512, dtype=bf), dev(2, 4, dtype=i64),
                                     dev(2, 16, 512), lse=dev(2, 8))
    torch.cuda.synchronize()
    assert bool((buf == 0).all())


def test_library_refusals_raise_indexer_error():
    wl = gen.config(2, scale=0.05)
    g = GpuWorkload(wl)
    note("library refusals through the binding")
    out = dev(wl.rows, 16, dtype=torch.int32, fill=-7)
    scores = dev(wl.rows, wl.max_row_len, fill=0)
    # k out of range
    with pytest.raises(dsa.IndexerError) as e:
        dsa.indexer_topk(scores, g.row_len, wl.max_row_len, 0, out)
    assert e.value.code == dsa.IDX_EINVAL and "k=0" in str(e.value)
    # a row longer than one chunk needs a workspace
    long_scores = dev(2, 1 << 17, fill=0)
    with pytest.raises(dsa.IndexerError) as e:
        dsa.indexer_topk(long_scores, i32([1 << 17, 5]), 1 << 17, 16, dev(2, 16, dtype=torch.int32))
    assert e.value.code == dsa.IDX_EWORKSPACE and "workspace" in str(e.value)
    # fp8 queries without their scales
    q8 = dev(wl.rows, 64, 128, dtype=torch.uint8, fill=0)
    with pytest.raises(dsa.IndexerError) as e:
        dsa.indexer_score(q8, g.w, g.cache, g.rows, scores)
    assert e.value.code == dsa.IDX_EINVAL and "q_scale" in str(e.value)
    # an unsupported head count for the attention
    kv = dev(64, 512, dtype=torch.bfloat16, fill=0)
    with pytest.raises(dsa.IndexerError) as e:
        dsa.indexer_sparse_attention(dev(2, 24, 512, dtype=torch.bfloat16), kv, dev(2, 4, dtype=torch.int64, fill=0),
                                     dev(2, 24, 512))
    assert e.value.code == dsa.IDX_EUNSUPPORTED and "heads" in str(e.value)
    # fp8 queries against bf16 keys
    gb = GpuWorkload(wl, key_dtype="bf16")
    with pytest.raises(dsa.IndexerError) as e:
        dsa.indexer_score(q8, g.w, gb.cache, gb.rows, scores, q_scale=dev(wl.rows, 64))
    assert e.value.code == dsa.IDX_EUNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == -7).all()) and bool((scores == 0).all())
