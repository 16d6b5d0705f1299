"""The Python binding's own argument checks, on a machine without a GPU: wrong dtypes,
host tensors, non-contiguous views and mismatched shapes are refused with TypeError or
ValueError before the library is called."""
import os

import pytest
import torch

import sparse_attention_token_store_amd as dsa

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="library not built")


def t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def test_host_tensors_and_dtypes_are_refused():
    # Each function checks its tensors in argument order (dtype, then contiguity,
    # then device), so with host tensors only the first tensor's checks are reached.
    bf, u8, i32, i64 = torch.bfloat16, torch.uint8, torch.int32, torch.int64
    with pytest.raises(ValueError, match="device tensor"):
        dsa.indexer_quant_fp8(t(4, 128, dtype=bf), t(4, 128, dtype=u8), t(4))
    with pytest.raises(TypeError, match="x"):
        dsa.indexer_quant_fp8(t(4, 128), t(4, 128, dtype=u8), t(4))
    with pytest.raises(TypeError, match="x"):
        dsa.index_k_store(t(4, 128), None, t(4, dtype=i64), None)
    with pytest.raises(TypeError, match="q"):
        dsa.indexer_q_prep(t(4, 64, 128), None, 0)
    with pytest.raises(TypeError, match="scores"):
        dsa.indexer_topk(t(2, 8, dtype=torch.float16), t(2, dtype=i32), 8, 4, t(2, 4, dtype=i32))
    with pytest.raises(ValueError, match="device tensor"):
        dsa.indexer_topk(t(2, 8), t(2, dtype=i32), 8, 4, t(2, 4, dtype=i32))
    with pytest.raises(TypeError, match="q must be bf16 or uint8"):
        dsa.indexer_score(t(1, 64, 128), t(1, 64), None, None, t(1, 8))
    with pytest.raises(TypeError, match="q must be bf16 or uint8"):
        dsa.indexer_score_topk(t(1, 64, 128), t(1, 64), None, None, 4, t(1, 4, dtype=i32), None)
    with pytest.raises(TypeError, match="idx"):
        dsa.indexer_translate(t(2, 4, dtype=i64), None, None, t(2, 4, dtype=i64))
    with pytest.raises(TypeError, match="q"):
        dsa.indexer_sparse_attention(t(1, 16, 512), t(8, 512, dtype=bf), t(1, 4, dtype=i64), t(1, 16, 512))
    with pytest.raises(TypeError, match="cache buffer"):
        dsa.kcache(t(1024, dtype=i32), dsa.IDX_FP8_E4M3, 64, 1)
    with pytest.raises(ValueError, match="cache buffer must be a device tensor"):
        dsa.kcache(torch.zeros(100, dtype=u8), dsa.IDX_FP8_E4M3, 64, 1)
    with pytest.raises(TypeError, match="block_table"):
        dsa.rows_desc(t(1, 4, dtype=i64), t(1, dtype=i32), t(1, dtype=i32), 100)


def test_non_contiguous_views_are_refused():
    scores = t(4, 16)[:, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        dsa.indexer_topk(scores, t(4, dtype=torch.int32), 8, 4, t(4, 4, dtype=torch.int32))


def test_sizes_and_workspaces_on_the_host():
    assert dsa.token_bytes(dsa.IDX_BF16) == 256
    assert dsa.token_bytes(dsa.IDX_FP8_E4M3) == 132
    assert dsa.token_bytes(dsa.IDX_MXFP4) == 68
    assert dsa.cache_bytes(dsa.IDX_FP8_E4M3, 64, 3) == 3 * 64 * 132
    assert dsa.workspace_bytes(dsa.IDX_OP_TOPK, 4, 20000, 512) == 0        # one level: no lists
    assert dsa.workspace_bytes(dsa.IDX_OP_TOPK, 4, 1 << 20, 1024) > 0
    assert dsa.workspace_bytes(dsa.IDX_OP_SCORE_TOPK, 4, 20000, 512) >= 4 * 20000 * 4
    assert dsa.attention_workspace_bytes(0, 512, 16) == 0
    assert dsa.abi_version() == 2
