"""Moving a synthetic workload onto the GPU through the library's own entry points
(the cache is filled by index_k_store), plus small torch<->numpy helpers."""
from __future__ import annotations

import sys

import numpy as np
import torch

import sparse_attention_token_store_amd as dsa


def note(msg: str):
    """Name the GPU step about to run (flushed, so a crash still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def i32(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def i64(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(dev)


def f32(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


class GpuWorkload:
    """Device copy of a workload: cache filled by the store, q, w, rows."""

    def __init__(self, wl, key_dtype: str | None = None, dev="cuda", fill=0xFF, block_table=None):
        self.wl = wl
        self.key_dtype = key_dtype or wl.key_dtype
        self.dtype = {"bf16": dsa.IDX_BF16, "fp8": dsa.IDX_FP8_E4M3, "fp4": dsa.IDX_MXFP4}[self.key_dtype]
        nbytes = dsa.cache_bytes(self.dtype, wl.block_size, wl.num_blocks)
        # unwritten slots hold 0xFF bytes (NaN codes / NaN bf16): masked positions must
        # never leak into a visible score
        self.buf = torch.full((nbytes,), fill, dtype=torch.uint8, device=dev)
        self.cache = dsa.kcache(self.buf, self.dtype, wl.block_size, wl.num_blocks)
        self.block_table = i32(wl.block_table if block_table is None else block_table, dev)
        self.row_seq = i32(wl.row_seq, dev)
        self.row_len = i32(wl.row_len, dev)
        self.rows = dsa.rows_desc(self.block_table, self.row_seq, self.row_len, wl.max_row_len)
        self.q = bf16_tensor(wl.q_bits, dev)
        self.w = f32(wl.w, dev)
        self.q_codes = self.q_scale = None
        x, slots = wl.prefix_tokens()
        self.prefix_x, self.prefix_slots = bf16_tensor(x, dev), i64(slots, dev)
        self.new_x = bf16_tensor(wl.new_x_bits, dev)
        self.new_pos = i32(wl.new_pos, dev)
        self.new_slots = i64(wl.new_slots(), dev)
        note(f"fill cache {wl.name} {self.key_dtype} bs={wl.block_size} tokens={x.shape[0]}")
        dsa.index_k_store(self.prefix_x, None, self.prefix_slots, self.cache, 0)
        torch.cuda.synchronize()

    def store_new(self, prequant=None):
        wl = self.wl
        if wl.new_x_bits.shape[0] == 0:
            return
        note(f"store chain {wl.name} n={wl.new_x_bits.shape[0]}")
        dsa.index_k_store(self.new_x, self.new_pos, self.new_slots, self.cache, dsa.IDX_STORE_ALL,
                          wl.rms_eps, wl.rope_base, wl.rope_dim, prequant_dbg=prequant)

    def quantise_q(self):
        note(f"quantise q {self.wl.name} rows={self.wl.rows}")
        self.q_codes = torch.empty(self.q.shape, dtype=torch.uint8, device=self.q.device)
        self.q_scale = torch.empty(self.q.shape[:2], dtype=torch.float32, device=self.q.device)
        dsa.indexer_quant_fp8(self.q, self.q_codes, self.q_scale)

    def query(self, use_fp8_q: bool):
        return (self.q_codes, self.q_scale) if use_fp8_q else (self.q, None)
