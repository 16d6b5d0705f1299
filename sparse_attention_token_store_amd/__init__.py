"""Python binding of libdsa_indexer.so (the C ABI in include/dsa_indexer.h).

Argument marshalling only: every step of the indexer runs in the library's HIP
kernels.  Tensors are torch tensors on the current HIP device; work is queued on
torch's current stream.  If the library has not been built the import fails loudly
(there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_indexer.so")

IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED, IDX_ELAUNCH, IDX_EWORKSPACE = 0, -1, -2, -3, -4
IDX_BF16, IDX_FP8_E4M3, IDX_MXFP4 = 1, 2, 3
IDX_STORE_RMSNORM, IDX_STORE_ROPE, IDX_STORE_HADAMARD = 1, 2, 4
IDX_STORE_ALL = 7
IDX_OP_TOPK, IDX_OP_SCORE_TOPK = 1, 2
IDX_STATIC_SCRATCH_BYTES = 32 << 20
HEAD_DIM = 128

EXPORTED = ("index_k_store", "indexer_q_prep", "indexer_quant_fp8", "indexer_score", "indexer_topk",
            "indexer_score_topk", "indexer_score_topk_static", "indexer_translate",
            "indexer_sparse_attention", "indexer_attention_workspace_bytes",
            "indexer_workspace_bytes", "indexer_last_error", "indexer_abi_version")
KV_DIM = 512


class IndexerError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class KCache(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int64)]


class Rows(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("row_seq", ctypes.c_void_p),
                ("row_len", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("max_row_len", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle; raises if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m sparse_attention_token_store_amd.build`")
    try:  # bind to the HIP runtime torch has loaded (torch ships its own copy)
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, i64, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                  ctypes.c_float, ctypes.c_size_t)
    sig = {
        "index_k_store": (i32, [vp, i64, vp, vp, KCache, u32, f32, f32, i32, vp, vp]),
        "indexer_q_prep": (i32, [vp, i64, i32, vp, u32, f32, f32, i32, vp, vp, vp, vp, vp]),
        "indexer_quant_fp8": (i32, [vp, i64, vp, vp, vp]),
        "indexer_score": (i32, [vp, i32, vp, vp, i32, KCache, Rows, vp, i64, vp]),
        "indexer_topk": (i32, [vp, i64, vp, i32, i32, i32, vp, vp, sz, vp]),
        "indexer_score_topk": (i32, [vp, i32, vp, vp, i32, KCache, Rows, i32, vp, vp, vp, vp, sz, vp]),
        "indexer_score_topk_static": (i32, [vp, i32, vp, vp, i32, KCache, Rows, i32, vp, vp, vp, vp]),
        "indexer_translate": (i32, [vp, i64, i32, KCache, Rows, vp, i64, vp]),
        "indexer_sparse_attention": (i32, [vp, i32, vp, i64, vp, i64, i32, i32, f32, vp, vp, vp, sz, vp]),
        "indexer_attention_workspace_bytes": (sz, [i32, i32, i32]),
        "indexer_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "indexer_last_error": (ctypes.c_char_p, []),
        "indexer_abi_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


# ------------------------------------------------------------------ marshalling

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, code):
    if code != IDX_OK:
        raise IndexerError(fn, code, load_library().indexer_last_error().decode())


def _need(t, dtype, name):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def kcache(buf, dtype: int, block_size: int, num_blocks: int) -> KCache:
    """Describe a paged cache held in the uint8 device tensor `buf`."""
    import torch
    _need(buf, torch.uint8, "cache buffer")
    per_block = block_size * token_bytes(dtype)
    if buf.numel() < per_block * num_blocks:
        raise ValueError("cache buffer smaller than num_blocks blocks")
    return KCache(buf.data_ptr(), dtype, block_size, num_blocks)


def token_bytes(dtype: int) -> int:
    """Cache bytes per token: bf16 256, fp8 128 codes + 4 scale, MXFP4 64 codes + 4 scales."""
    return {IDX_BF16: 256, IDX_FP8_E4M3: 132, IDX_MXFP4: 68}[dtype]


def cache_bytes(dtype: int, block_size: int, num_blocks: int) -> int:
    return block_size * token_bytes(dtype) * num_blocks


def rows_desc(block_table, row_seq, row_len, max_row_len: int) -> Rows:
    import torch
    for t, n in ((block_table, "block_table"), (row_seq, "row_seq"), (row_len, "row_len")):
        _need(t, torch.int32, n)
    return Rows(block_table.data_ptr(), block_table.shape[1], block_table.shape[0],
                row_seq.data_ptr(), row_len.data_ptr(), row_len.shape[0], int(max_row_len))


def workspace_bytes(op: int, rows: int, max_row_len: int, k: int) -> int:
    return int(load_library().indexer_workspace_bytes(op, rows, max_row_len, k))


def abi_version() -> int:
    return int(load_library().indexer_abi_version())


# ------------------------------------------------------------------ entry points

def index_k_store(x, positions, slot_mapping, cache: KCache, flags: int = 0, rms_eps: float = 1e-6,
                  rope_base: float = 10000.0, rope_dim: int = 64, prequant_dbg=None, stream=None):
    import torch
    _need(x, torch.bfloat16, "x")
    _need(positions, torch.int32, "positions")
    _need(slot_mapping, torch.int64, "slot_mapping")
    _need(prequant_dbg, torch.float32, "prequant_dbg")
    n = x.shape[0]
    if x.shape[-1] != HEAD_DIM or slot_mapping.shape[0] != n:
        raise ValueError("x must be [n,128] and slot_mapping [n]")
    _check("index_k_store", load_library().index_k_store(
        _ptr(x), n, _ptr(positions), _ptr(slot_mapping), cache, flags, rms_eps, rope_base, rope_dim,
        _ptr(prequant_dbg), _stream(stream)))


def indexer_q_prep(q, positions, flags: int, rope_base: float = 10000.0, rope_dim: int = 64,
                   out_bf16=None, codes=None, scales=None, rms_eps: float = 1e-6, prequant_dbg=None,
                   stream=None):
    """q: bf16 [rows, heads, 128]; positions: int32 [rows] (needed with IDX_STORE_ROPE)."""
    import torch
    _need(q, torch.bfloat16, "q")
    _need(positions, torch.int32, "positions")
    _need(out_bf16, torch.bfloat16, "out_bf16")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float32, "scales")
    _need(prequant_dbg, torch.float32, "prequant_dbg")
    if q.dim() != 3 or q.shape[-1] != HEAD_DIM:
        raise ValueError("q must be [rows, heads, 128]")
    rows, heads = q.shape[0], q.shape[1]
    n_vec = rows * heads
    for t, n, want in ((out_bf16, "out_bf16", n_vec * HEAD_DIM), (codes, "codes", n_vec * HEAD_DIM),
                       (scales, "scales", n_vec), (prequant_dbg, "prequant_dbg", n_vec * HEAD_DIM)):
        if t is not None and t.numel() != want:
            raise ValueError(f"{n} must hold {want} elements")
    if positions is not None and positions.numel() != rows:
        raise ValueError("positions must hold one entry per row")
    _check("indexer_q_prep", load_library().indexer_q_prep(
        _ptr(q), n_vec, heads, _ptr(positions), flags, rms_eps, rope_base, rope_dim, _ptr(out_bf16),
        _ptr(codes), _ptr(scales), _ptr(prequant_dbg), _stream(stream)))


def indexer_quant_fp8(x, codes, scales, stream=None):
    import torch
    _need(x, torch.bfloat16, "x")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float32, "scales")
    n_vec = x.numel() // HEAD_DIM
    if codes.numel() != x.numel() or scales.numel() != n_vec:
        raise ValueError("codes must match x and scales must have x.numel()/128 entries")
    _check("indexer_quant_fp8", load_library().indexer_quant_fp8(
        _ptr(x), n_vec, _ptr(codes), _ptr(scales), _stream(stream)))


def _q_args(q, q_scale, w):
    import torch
    if q.dtype == torch.bfloat16:
        q_dtype = IDX_BF16
    elif q.dtype == torch.uint8:
        q_dtype = IDX_FP8_E4M3
        _need(q_scale, torch.float32, "q_scale")
    else:
        raise TypeError("q must be bf16 or uint8 e4m3 codes")
    _need(q, q.dtype, "q")
    _need(w, torch.float32, "w")
    return q_dtype, q.shape[1]


def indexer_score(q, w, cache: KCache, rows: Rows, scores, q_scale=None, stream=None):
    import torch
    q_dtype, heads = _q_args(q, q_scale, w)
    _need(scores, torch.float32, "scores")
    _check("indexer_score", load_library().indexer_score(
        _ptr(q), q_dtype, _ptr(q_scale), _ptr(w), heads, cache, rows, _ptr(scores),
        scores.shape[1], _stream(stream)))


def indexer_topk(scores, row_len, max_row_len: int, k: int, out_idx, ws=None, stream=None):
    import torch
    _need(scores, torch.float32, "scores")
    _need(row_len, torch.int32, "row_len")
    _need(out_idx, torch.int32, "out_idx")
    rows = row_len.shape[0]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("indexer_topk", load_library().indexer_topk(
        _ptr(scores), scores.shape[1], _ptr(row_len), rows, max_row_len, k, _ptr(out_idx),
        _ptr(ws), nbytes, _stream(stream)))


def indexer_score_topk(q, w, cache: KCache, rows: Rows, k: int, out_idx, ws, out_scores=None,
                       q_scale=None, out_slots=None, stream=None):
    import torch
    q_dtype, heads = _q_args(q, q_scale, w)
    _need(out_idx, torch.int32, "out_idx")
    _need(out_scores, torch.float32, "out_scores")
    _need(out_slots, torch.int64, "out_slots")
    if out_slots is not None and out_slots.numel() < out_idx.numel():
        raise ValueError("out_slots must hold [rows, k] entries")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("indexer_score_topk", load_library().indexer_score_topk(
        _ptr(q), q_dtype, _ptr(q_scale), _ptr(w), heads, cache, rows, k, _ptr(out_idx),
        _ptr(out_slots), _ptr(out_scores), _ptr(ws), nbytes, _stream(stream)))


def indexer_score_topk_static(q, w, cache: KCache, rows: Rows, k: int, out_idx, out_scores=None,
                              q_scale=None, out_slots=None, stream=None):
    """indexer_score_topk with the library's static per-GPU scratch instead of a
    workspace (nothing is allocated; overlapping calls on one GPU race)."""
    import torch
    q_dtype, heads = _q_args(q, q_scale, w)
    _need(out_idx, torch.int32, "out_idx")
    _need(out_scores, torch.float32, "out_scores")
    _need(out_slots, torch.int64, "out_slots")
    if out_slots is not None and out_slots.numel() < out_idx.numel():
        raise ValueError("out_slots must hold [rows, k] entries")
    _check("indexer_score_topk_static", load_library().indexer_score_topk_static(
        _ptr(q), q_dtype, _ptr(q_scale), _ptr(w), heads, cache, rows, k, _ptr(out_idx),
        _ptr(out_slots), _ptr(out_scores), _stream(stream)))


def indexer_translate(idx, cache: KCache, rows: Rows, out_slots, stream=None):
    """Physical cache slots of the index lists idx [rows, k] (int32) into out_slots
    [rows, k] (int64); -1 wherever an entry addresses no visible key."""
    import torch
    _need(idx, torch.int32, "idx")
    _need(out_slots, torch.int64, "out_slots")
    if idx.dim() != 2 or tuple(out_slots.shape) != tuple(idx.shape) or idx.shape[0] != rows.rows:
        raise ValueError("idx and out_slots must both be [rows, k]")
    _check("indexer_translate", load_library().indexer_translate(
        _ptr(idx), idx.shape[1], idx.shape[1], cache, rows, _ptr(out_slots), out_slots.shape[1],
        _stream(stream)))


def indexer_sparse_attention(q, kv, slots, out, k=None, scale=None, lse=None, ws=None, stream=None):
    """q: bf16 [rows, heads, 512]; kv: bf16 [num_slots, 512] (the main KV cache seen
    as slots); slots: int64 [rows, ld] (the first k entries of a row are its list,
    negative entries padding); out: fp32 [rows, heads, 512]; lse: optional fp32
    [rows, heads]; scale defaults to 1/sqrt(512); ws: alloc_attention_workspace()."""
    import torch
    _need(q, torch.bfloat16, "q")
    _need(kv, torch.bfloat16, "kv")
    _need(slots, torch.int64, "slots")
    _need(out, torch.float32, "out")
    _need(lse, torch.float32, "lse")
    if q.dim() != 3 or q.shape[-1] != KV_DIM or kv.dim() != 2 or kv.shape[-1] != KV_DIM:
        raise ValueError("q must be [rows, heads, 512] and kv [num_slots, 512]")
    rows, heads = q.shape[0], q.shape[1]
    if slots.dim() != 2 or slots.shape[0] != rows or tuple(out.shape) != tuple(q.shape):
        raise ValueError("slots must be [rows, ld] and out [rows, heads, 512]")
    if lse is not None and tuple(lse.shape) != (rows, heads):
        raise ValueError("lse must be [rows, heads]")
    k = slots.shape[1] if k is None else int(k)
    scale = KV_DIM ** -0.5 if scale is None else float(scale)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("indexer_sparse_attention", load_library().indexer_sparse_attention(
        _ptr(q), heads, _ptr(kv), kv.shape[0], _ptr(slots), slots.shape[1], k, rows, scale, _ptr(out),
        _ptr(lse), _ptr(ws), nbytes, _stream(stream)))


def attention_workspace_bytes(rows: int, k: int, heads: int) -> int:
    return int(load_library().indexer_attention_workspace_bytes(rows, k, heads))


def _aligned_bytes(n: int, device):
    import torch
    if n == 0:
        return None
    t = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + n]


def alloc_attention_workspace(rows: int, k: int, heads: int, device="cuda"):
    """A 256-byte aligned workspace for indexer_sparse_attention (or None)."""
    return _aligned_bytes(attention_workspace_bytes(rows, k, heads), device)


def alloc_workspace(op: int, rows: int, max_row_len: int, k: int, device="cuda"):
    """A 256-byte aligned uint8 workspace tensor of the size the op needs (or None)."""
    return _aligned_bytes(workspace_bytes(op, rows, max_row_len, k), device)
