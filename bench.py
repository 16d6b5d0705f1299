#!/usr/bin/env python3
"""Benchmark of the DSA indexer hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input, with every
input already resident in HBM:
  decode workloads   index_k_store of the step's new tokens (RMSNorm -> RoPE ->
                     Hadamard -> fp8 -> paged scatter), indexer_score over the
                     paged cache, indexer_topk of every row
  prefill workload   indexer_quant_fp8 of the queries, indexer_score (fp8 x fp8),
                     indexer_topk
These are exactly the kernels indexer_score_topk chains; calling the entry points
separately lets HIP events on the launch stream time each kernel inside the timed
region.  Key caches are replicated and rotated so that every step reads its keys
from HBM, not from the 256 MB last-level cache.

Timing: the K timed steps are queued behind a device-side delay, so the GPU runs
them back to back whatever the host's launch rate; HIP events on the launch stream
bracket the region and every kernel in it.  A second, host-paced pass (no delay)
is reported beside it.  The pass with events around every kernel also gives the
p10 / median / p90 of the step and of each kernel (`kernel_ms.p10_p50_p90`).  The
default is 100 timed steps after 10 warm-up steps.

Default run: the headline line is the chunked prefill (4096 query rows on a
32,768-token prefix, 142.6M visible (query, key) pairs per step, the largest
configuration), and `per_config` holds the same measurements for the tiny decode,
decode batch 32, the A/B decode with bf16 and with fp8 keys, and the long decode.
Every entry reports the dominant kernel's roofline fraction (kernel time only) and
the score + top-k step fraction, each against the vendor peak and against the peak
measured in the same run (`peaks_measured`), and the CPU oracle on a bounded sample.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer keys scored/s + top-k selections/s at 1 GPU; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
COLD_BYTES = 640 << 20          # replicas of the key cache cover at least this much

WORKLOADS = {
    # name: (config, key dtype, description)
    "tiny_decode": (1, "bf16", "decode 1 x 2000, bf16 keys, top-512"),
    "decode_b32": (2, "fp8", "decode batch 32, S~U[4500,22000], fp8 keys, top-512"),
    "ab_bf16": (3, "bf16", "decode 16 x 131072, bf16 keys, top-1024"),
    "ab_fp8": (3, "fp8", "decode 16 x 131072, fp8 keys, top-1024"),
    "ab_fp4": (3, "fp4", "decode 16 x 131072, MXFP4 keys (e2m1 + e8m0 per 32), top-1024"),
    "prefill": (4, "fp8", "chunked prefill 4096 rows on a 32768 prefix, fp8 keys, top-1024"),
    "prefill_fp4": (4, "fp4", "chunked prefill 4096 rows on a 32768 prefix, MXFP4 keys, top-1024"),
    "long_decode": (5, "fp8", "decode 4 x 1048576 fp8 keys after a 4096-token store, top-1024"),
}
HEADLINE = "prefill"
PER_CONFIG = ["tiny_decode", "decode_b32", "ab_bf16", "ab_fp8", "long_decode"]
KEY_BYTES = {"fp8": 132, "fp4": 68, "bf16": 256}


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_attention_token_store_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"score_decode": ["score_decode.hip", "common.hpp"],
                  "score_prefill": ["score_prefill.hip", "common.hpp"],
                  "q_prep": ["store.hip", "common.hpp"],
                  "translate": ["topk.hip", "common.hpp"],
                  "sparse_attention": ["attention.hip", "common.hpp"]}


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if the summary in
    profiles/ was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return float(m.group(1))


class Event:
    """A HIP timing event without the system-scope fence of a default event (see
    dsa_bench_event_create); read after the stream has been synchronised."""

    def __init__(self, probes):
        self.p = probes
        self.h = probes.lib.dsa_bench_event_create()
        if not self.h:
            raise RuntimeError("dsa_bench_event_create failed")

    def record(self):
        if self.p.lib.dsa_bench_event_record(ctypes.c_void_p(self.h), self.p.stream()) != 0:
            raise RuntimeError("dsa_bench_event_record failed")

    def ms_to(self, other) -> float:
        ms = self.p.lib.dsa_bench_event_ms(ctypes.c_void_p(self.h), ctypes.c_void_p(other.h))
        if ms < 0:
            raise RuntimeError("dsa_bench_event_ms failed")
        return float(ms)

    def __del__(self):
        try:
            self.p.lib.dsa_bench_event_destroy(ctypes.c_void_p(self.h))
        except Exception:
            pass


class Probes:
    """The measurement kernels of libdsa_bench.so: a device-side delay, a streaming
    read, the dense MFMA rate kernels, and fence-free timing events."""

    def __init__(self):
        import torch
        path = os.path.join(ROOT, "sparse_attention_token_store_amd", "libdsa_bench.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built: run `python -m sparse_attention_token_store_amd.build`")
        self.torch = torch
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.dsa_bench_spin.argtypes = [ctypes.c_double, vp]
        lib.dsa_bench_stream_read.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_int, vp]
        lib.dsa_bench_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                       ctypes.POINTER(ctypes.c_double), vp]
        for f in (lib.dsa_bench_spin, lib.dsa_bench_stream_read, lib.dsa_bench_mfma):
            f.restype = ctypes.c_int
        lib.dsa_bench_event_create.argtypes, lib.dsa_bench_event_create.restype = [], vp
        lib.dsa_bench_event_record.argtypes, lib.dsa_bench_event_record.restype = [vp, vp], ctypes.c_int
        lib.dsa_bench_event_ms.argtypes, lib.dsa_bench_event_ms.restype = [vp, vp], ctypes.c_float
        lib.dsa_bench_event_destroy.argtypes, lib.dsa_bench_event_destroy.restype = [vp], None
        self.lib = lib
        self.sink = torch.zeros(4, dtype=torch.float32, device="cuda")

    def stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def event(self) -> Event:
        return Event(self)

    def spin(self, us: float):
        if self.lib.dsa_bench_spin(float(us), self.stream()) != 0:
            raise RuntimeError("dsa_bench_spin failed")

    def _timed(self, fn, reps=5):
        best = None
        for _ in range(reps):
            a, b = self.event(), self.event()
            a.record()
            fn()
            b.record()
            self.torch.cuda.synchronize()
            ms = a.ms_to(b)
            best = ms if best is None else min(best, ms)
        return best

    def peaks(self) -> dict:
        """Best of 5 launches each, over a few grid sizes: a 2 GiB streaming read, and
        the fp8 and bf16 MFMA rate kernels (4 wavefronts per workgroup)."""
        torch = self.torch
        nbytes = 2 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        s = ctypes.c_void_p(self.sink.data_ptr())
        best_rd, best_blocks = None, None
        for blocks in (1024, 2048, 4096, 8192):
            def rd():
                if self.lib.dsa_bench_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, s, blocks, self.stream()):
                    raise RuntimeError("dsa_bench_stream_read failed")
            rd()
            ms = self._timed(rd)
            if best_rd is None or ms < best_rd:
                best_rd, best_blocks = ms, blocks
        del buf
        out = {"hbm_read_GBs": nbytes / (best_rd / 1e3) / 1e9,
               "hbm_read_note": (f"2 GiB streaming read, 16-byte non-temporal loads, 8 in flight per thread, "
                                 f"best of 5 at the best of 1024-8192 workgroups ({best_blocks})")}
        for name, fp8, iters in (("fp8_mfma_TFLOPs", 1, 1000), ("bf16_mfma_TFLOPs", 0, 2000)):
            best = 0.0
            for blocks in (1024, 2048):
                fl = ctypes.c_double(0)

                def mm():
                    if self.lib.dsa_bench_mfma(fp8, blocks, iters, s, ctypes.byref(fl), self.stream()):
                        raise RuntimeError("dsa_bench_mfma failed")
                mm()
                ms = self._timed(mm)
                best = max(best, fl.value / (ms / 1e3) / 1e12)
            out[name] = best
        out["mfma_note"] = ("16 independent accumulators per wavefront, 4 or 8 wavefronts per SIMD, best of "
                            "5; fp8: v_mfma_scale_f32_16x16x128_f8f6f4, bf16: v_mfma_f32_16x16x32_bf16")
        torch.cuda.empty_cache()
        return out


class Runner:
    def __init__(self, name: str, replicas: int | None, wl=None):
        import torch
        import sparse_attention_token_store_amd as dsa
        from synth import gen
        self.torch, self.dsa, self.name = torch, dsa, name
        cfg, kd, self.desc = WORKLOADS[name]
        wl = wl if wl is not None else gen.config(cfg, key_dtype=kd)
        self.wl, self.kd = wl, kd
        dev = "cuda"
        self.dtype = {"bf16": dsa.IDX_BF16, "fp8": dsa.IDX_FP8_E4M3, "fp4": dsa.IDX_MXFP4}[kd]
        cbytes = dsa.cache_bytes(self.dtype, wl.block_size, wl.num_blocks)
        self.replicas = replicas or max(1, -(-COLD_BYTES // cbytes))

        def t_bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        def t(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)

        x, slots = wl.prefix_tokens()
        x_t, slots_t = t_bf16(x), t(slots, np.int64)
        self.bufs, self.caches = [], []
        for _ in range(self.replicas):
            b = torch.empty(cbytes, dtype=torch.uint8, device=dev)
            c = dsa.kcache(b, self.dtype, wl.block_size, wl.num_blocks)
            dsa.index_k_store(x_t, None, slots_t, c, 0)
            self.bufs.append(b)
            self.caches.append(c)
        del x_t, slots_t
        self.block_table = t(wl.block_table, np.int32)
        self.row_seq, self.row_len = t(wl.row_seq, np.int32), t(wl.row_len, np.int32)
        self.rows = dsa.rows_desc(self.block_table, self.row_seq, self.row_len, wl.max_row_len)
        self.q = t_bf16(wl.q_bits)
        self.w = t(wl.w, np.float32)
        self.new_x, self.new_pos = t_bf16(wl.new_x_bits), t(wl.new_pos, np.int32)
        self.new_slots = t(wl.new_slots(), np.int64)
        self.prefill = wl.q_dtype == "fp8"
        if self.prefill:
            self.q_codes = torch.empty(self.q.shape, dtype=torch.uint8, device=dev)
            self.q_scale = torch.empty(self.q.shape[:2], dtype=torch.float32, device=dev)
        self.ld = -(-wl.max_row_len // 64) * 64
        self.scores = torch.empty((wl.rows, self.ld), dtype=torch.float32, device=dev)
        self.out_idx = torch.empty((wl.rows, wl.k), dtype=torch.int32, device=dev)
        self.ws = dsa.alloc_workspace(dsa.IDX_OP_TOPK, wl.rows, wl.max_row_len, wl.k)
        torch.cuda.synchronize()

    def step(self, i, ev=None):
        """One pass of the hot path on replica i % R.  ev: optional list of 4 events
        recorded before the store / query quantisation, before and after the score
        kernel, and after the top-k."""
        dsa, wl = self.dsa, self.wl
        cache = self.caches[i % self.replicas]
        if ev:
            ev[0].record()
        if wl.new_x_bits.shape[0]:
            dsa.index_k_store(self.new_x, self.new_pos, self.new_slots, cache, dsa.IDX_STORE_ALL,
                              wl.rms_eps, wl.rope_base, wl.rope_dim)
        if self.prefill:
            dsa.indexer_quant_fp8(self.q, self.q_codes, self.q_scale)
        if ev:
            ev[1].record()
        if self.prefill:
            dsa.indexer_score(self.q_codes, self.w, cache, self.rows, self.scores, q_scale=self.q_scale)
        else:
            dsa.indexer_score(self.q, self.w, cache, self.rows, self.scores)
        if ev:
            ev[2].record()
        dsa.indexer_topk(self.scores, self.row_len, wl.max_row_len, wl.k, self.out_idx, self.ws)
        if ev:
            ev[3].record()

    # algorithmic work of the dominant (score) kernel per launch
    def score_work(self):
        wl = self.wl
        keys = wl.visible_keys
        if self.prefill:
            flops = 2.0 * wl.heads * 128 * keys
            return {"bound": "mfma", "unit": "TFLOP/s", "work": flops, "peak": FP8_MFMA_PEAK_TFLOPS,
                    "kernel": "score_prefill", "peak_key": "fp8_mfma_TFLOPs",
                    "per_unit": "16,384 FLOP per visible (row, key) pair (64 heads x 128 x 2)"}
        key_bytes = KEY_BYTES[self.kd]
        per_key = key_bytes + 4 + 4.0 / wl.block_size          # key, score write, table entry
        per_row = wl.heads * 128 * 2 + wl.heads * 4 + 8         # q (bf16), w, row_seq + row_len
        pad = sum(wl.max_row_len - int(n) for n in wl.row_len) * 4   # -inf padding writes
        nbytes = keys * per_key + wl.rows * per_row + pad
        return {"bound": "hbm", "unit": "GB/s", "work": nbytes, "peak": HBM_PEAK_GBS,
                "kernel": "score_decode", "peak_key": "hbm_read_GBs",
                "per_unit": f"{key_bytes} B per visible key + 4 B score + {4.0 / wl.block_size:g} B table "
                            f"entry; {per_row} B per row (q, w, row data)"}

    # algorithmic work of scoring plus top-k as one fused step: no intermediate scores
    def score_topk_work(self):
        wl = self.wl
        keys = wl.visible_keys
        if self.prefill:
            return 2.0 * wl.heads * 128 * keys
        key_bytes = KEY_BYTES[self.kd]
        q_bytes = wl.heads * 128 * 2
        return (keys * (key_bytes + 4.0 / wl.block_size) + wl.rows * (q_bytes + wl.heads * 4 + 8)
                + wl.rows * wl.k * 4)


def bench_q_prep(args, run):
    """Time indexer_q_prep on the workload's query tensor [rows][64][128]: interleaved
    RoPE on the trailing 64 dims at each row's position, the Hadamard rotation and
    fp8 quantisation (codes + per-vector scale), the query side of the path.  One
    launch per step; HIP events on the launch stream bracket the timed steps."""
    torch, dsa, wl = run.torch, run.dsa, run.wl
    rows, heads = wl.q_bits.shape[0], wl.q_bits.shape[1]
    pos = torch.from_numpy((np.asarray(wl.row_len, np.int64) - 1).astype(np.int32)).cuda()
    codes = torch.empty(run.q.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    flags = dsa.IDX_STORE_ROPE | dsa.IDX_STORE_HADAMARD

    def launch():
        dsa.indexer_q_prep(run.q, pos, flags, wl.rope_base, wl.rope_dim, codes=codes, scales=scales)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        launch()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    n_vec = rows * heads
    nbytes = n_vec * (256 + 128 + 4) + rows * 4      # q in, codes + scale out, positions
    achieved = nbytes / (ms / 1e3) / 1e9
    return {
        "metric": "query vectors prepared/s (RoPE + Hadamard + fp8) at 1 GPU",
        "value": n_vec / (ms / 1e3),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} queries", "rows": rows, "heads": heads, "head_dim": 128,
                   "rope_dim": wl.rope_dim, "rope_base": wl.rope_base, "flags": "rope|hadamard",
                   "output": "fp8 e4m3 codes + fp32 scale", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "q_prep", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile("q_prep", args.workload),
                     "algorithmic_per_launch": nbytes},
    }


def bench_attention(probes, steps, warmup, heads, rows=32, k=512, num_slots=423936, lists=64):
    """indexer_sparse_attention of `heads` query heads over `k` selected slots per row
    (decode batch 32 at top-512: the slot space of the decode-batch KV cache, 512-dim
    bf16 states, 434 MB), each step with a fresh list of distinct random slots (64
    lists rotate, 1 GB of KV rows touched, so the gathers come from HBM).  Queued
    ahead behind a device delay; fence-free events bracket the timed launches."""
    import torch
    import sparse_attention_token_store_amd as dsa
    from synth import gen
    rng = np.random.default_rng(1)
    gen_t = torch.Generator(device="cuda").manual_seed(3)
    kv = torch.randn((num_slots, 512), dtype=torch.bfloat16, device="cuda", generator=gen_t)
    q_bits, _ = gen.attention_case(rows, heads, 1, 1, seed=2)
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    sl = torch.from_numpy(np.stack([np.stack([rng.choice(num_slots, k, replace=False) for _ in range(rows)])
                                    for _ in range(lists)]).astype(np.int64)).cuda()
    out = torch.empty((rows, heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    ws = dsa.alloc_attention_workspace(rows, k, heads)

    def launch(i):
        dsa.indexer_sparse_attention(q, kv, sl[i % lists], out, lse=lse, ws=ws)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    a, b = probes.event(), probes.event()
    probes.spin(min(200_000.0, 2000.0 + 100.0 * steps))
    a.record()
    for i in range(steps):
        launch(warmup + i)
    b.record()
    torch.cuda.synchronize()
    ms = a.ms_to(b) / steps
    nbytes = rows * k * 1024 + rows * heads * 1024 + rows * heads * (512 * 4 + 4) + rows * k * 8
    achieved = nbytes / (ms / 1e3) / 1e9
    splits_ws = dsa.attention_workspace_bytes(rows, k, heads)
    del kv, sl
    torch.cuda.empty_cache()
    traffic = traffic_from_profile("sparse_attention", f"decode_b32_h{heads}") \
        if (rows, k, num_slots) == (32, 512, 423936) else None
    return {"workload": f"sparse attention, {rows} rows x top-{k} slots, {heads} heads x 512, bf16 KV",
            "ms_per_launch": ms, "rows_per_s": rows / (ms / 1e3),
            "kv_rows_per_s": rows * k / (ms / 1e3), "heads": heads, "rows": rows, "k": k,
            "split_workspace_bytes": splits_ws,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "algorithmic_per_launch": nbytes,
                         "traffic": traffic,
                         "algorithmic_per_unit": "1024 B per listed KV row + 8 B slot; per row and head "
                                                 "1 KB of q, 2 KB of fp32 output, 4 B of lse"}}


def bench_translate(args, run):
    """Time indexer_translate on selections shaped like the step's top-k output
    (k sorted distinct visible positions per row, -1 padding on short rows), and the
    cost the fused slots add to indexer_score_topk (same call with and without
    out_slots, on the same stream, alternating)."""
    torch, dsa, wl = run.torch, run.dsa, run.wl
    rng = np.random.default_rng(0)
    k = wl.k
    sel = np.full((wl.rows, k), -1, np.int32)
    for r in range(wl.rows):
        n = int(wl.row_len[r])
        m = min(n, k)
        sel[r, :m] = np.sort(rng.choice(n, m, replace=False))
    idx = torch.from_numpy(sel).cuda()
    slots = torch.empty((wl.rows, k), dtype=torch.int64, device="cuda")
    cache = run.caches[0]

    def timed(fn, steps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms = timed(lambda: dsa.indexer_translate(idx, cache, run.rows, slots), args.steps)
    # fused: the whole score + top-k with and without the slots output
    q, qs = (run.q_codes, run.q_scale) if run.prefill else (run.q, None)
    if run.prefill:
        dsa.indexer_quant_fp8(run.q, run.q_codes, run.q_scale)
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
    out = torch.empty((wl.rows, k), dtype=torch.int32, device="cuda")
    fsteps = max(3, min(args.steps, 50))
    plain, fused = [], []
    for _ in range(3):
        plain.append(timed(lambda: dsa.indexer_score_topk(q, run.w, cache, run.rows, k, out, ws, q_scale=qs), fsteps))
        fused.append(timed(lambda: dsa.indexer_score_topk(q, run.w, cache, run.rows, k, out, ws, q_scale=qs,
                                                          out_slots=slots), fsteps))
    n = wl.rows * k
    table_bytes = int(wl.block_table.size) * 4
    nbytes = n * (4 + 8) + table_bytes + wl.rows * 8
    achieved = nbytes / (ms / 1e3) / 1e9
    return {
        "metric": "selected indices translated to physical slots/s at 1 GPU",
        "value": n / (ms / 1e3),
        "unit": "indices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} selections", "rows": wl.rows, "k": k,
                   "block_size": wl.block_size, "parallelism": "single GPU"},
        "fused_in_score_topk": {"ms_without_slots": float(np.median(plain)),
                                "ms_with_slots": float(np.median(fused)),
                                "added_ms": float(np.median(fused) - np.median(plain))},
        "roofline": {"bound": "hbm", "kernel": "translate", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile("translate", args.workload),
                     "algorithmic_per_launch": nbytes},
    }



def cpu_info() -> dict:
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    try:
        import threadpoolctl
        blas = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        blas = None
    return {"cpu_model": model, "affinity_cores": affinity, "blas_threads": blas}


def cpu_baseline(wl, kd, budget_s=12.0, min_s=None):
    """The oracle (numpy float64, BLAS threads as configured) on a bounded sample of
    the same workload: whole rows (store chain of the row's new tokens, key
    dequantisation, query quantisation for fp8 queries, score, top-k), repeated over
    the rows until about budget_s of CPU work has been timed."""
    from oracle import oracle as O
    min_s = budget_s * 0.7 if min_s is None else min_s
    info = cpu_info()
    rows_done, keys_done, t_total = 0, 0, 0.0
    order = np.argsort(wl.row_len)[::-1] if wl.rows > 1 else np.arange(wl.rows)
    prefix_cache = {}
    passes = 0
    while t_total < min_s:
        for r in order:
            b = int(wl.row_seq[r])
            n = int(wl.row_len[r])
            if b not in prefix_cache:               # cache fill: not timed (setup)
                x = wl.keys_bits[b]
                if kd == "fp8":
                    prefix_cache[b] = O.quant_fp8(O.bf16_bits_to_f32(x))
                elif kd == "fp4":
                    prefix_cache[b] = O.quant_mxfp4(O.bf16_bits_to_f32(x))
                else:
                    prefix_cache[b] = x
            t0 = time.perf_counter()
            sel = wl.new_seq == b
            parts = []
            store = prefix_cache[b]
            nstored = int(wl.stored_len[b])
            for p0 in range(0, min(n, nstored), 1 << 16):
                p1 = min(n, nstored, p0 + (1 << 16))
                if kd == "fp8":
                    parts.append(O.dequant_fp8(store[0][p0:p1], store[1][p0:p1]))
                elif kd == "fp4":
                    parts.append(O.dequant_mxfp4(store[0][p0:p1], store[1][p0:p1]))
                else:
                    parts.append(O.bf16_bits_to_f64(store[p0:p1]))
            if n > nstored:
                y = O.store_chain(wl.new_x_bits[sel], wl.new_pos[sel], 7, wl.rms_eps, wl.rope_base, wl.rope_dim)
                if kd == "fp8":
                    parts.append(O.dequant_fp8(*O.quant_fp8(y.astype(np.float32))))
                elif kd == "fp4":
                    parts.append(O.dequant_mxfp4(*O.quant_mxfp4(y.astype(np.float32))))
                else:
                    parts.append(O.bf16_bits_to_f64(O.bf16_round(y)))
            keys = np.concatenate(parts, 0)[:n]
            q = O.bf16_bits_to_f64(wl.q_bits[r])
            if wl.q_dtype == "fp8":
                c, s = O.quant_fp8(O.bf16_bits_to_f32(wl.q_bits[r]))
                q = O.dequant_fp8(c, s)
            sc = O.score(q, wl.w[r].astype(np.float64), keys)
            O.topk(sc[None], [n], wl.k)
            t_total += time.perf_counter() - t0
            rows_done += 1
            keys_done += n
            if t_total >= budget_s:
                break
        passes += 1
    return {"value": keys_done / t_total, "unit": "keys/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"{rows_done} rows ({keys_done} visible keys; {passes} pass(es) over the "
                      f"{wl.rows} rows of the same workload), {t_total:.1f} s: store chain of the "
                      f"row's new tokens, key decode, query quantisation (fp8 queries), float64 score, "
                      f"sort-based top-k",
            "selections_per_s": rows_done / t_total, **info}


def time_steps(run, probes, steps, warmup, queue_ahead=True, per_kernel=False, warm=False):
    """Run `warmup` untimed steps, then time `steps` steps between two events.  With
    queue_ahead the steps are queued behind a device-side delay long enough for the
    host to queue them all, so the GPU runs them back to back.  With per_kernel each
    step also records events around its kernels.  With warm every step reads the
    first key-cache replica (cache-resident where it fits) instead of rotating.
    Returns (ms per step, mean kernel ms {store_or_quant, score, topk} or None)."""
    torch = run.torch
    rep = (lambda i: 0) if warm else (lambda i: i)
    for i in range(warmup):
        run.step(rep(i))
    torch.cuda.synchronize()
    evs = [[probes.event() for _ in range(4)] for _ in range(steps)] if per_kernel else None
    t_start, t_end = probes.event(), probes.event()
    torch.cuda.synchronize()
    if queue_ahead:
        probes.spin(min(200_000.0, 2000.0 + 400.0 * steps))
    t_start.record()
    for i in range(steps):
        run.step(rep(i), evs[i] if evs else None)
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.ms_to(t_end) / steps
    if not evs:
        return ms, None
    k = {"store_or_quant": float(np.mean([e[0].ms_to(e[1]) for e in evs])),
         "score": float(np.mean([e[1].ms_to(e[2]) for e in evs])),
         "topk": float(np.mean([e[2].ms_to(e[3]) for e in evs]))}
    # p10 / median / p90 over the steps of this pass: each step between its own first
    # and last event, and each kernel between the events around it
    pct = lambda xs: [float(v) for v in np.percentile(xs, [10, 50, 90])]
    k["p10_p50_p90"] = {"step": pct([e[0].ms_to(e[3]) for e in evs]),
                        "store_or_quant": pct([e[0].ms_to(e[1]) for e in evs]),
                        "score": pct([e[1].ms_to(e[2]) for e in evs]),
                        "topk": pct([e[2].ms_to(e[3]) for e in evs]),
                        "steps": steps}
    return ms, k


def measure(name, args, probes, peaks, wl=None, cpu_budget=None) -> dict:
    """Every figure of one workload: step time, kernel times, roofline fractions,
    the host-paced step time and the CPU oracle."""
    torch = probes.torch
    run = Runner(name, args.replicas, wl=wl)
    wl = run.wl
    print(f"[bench] {name}: {run.desc}; rows={wl.rows} visible_keys={wl.visible_keys} "
          f"replicas={run.replicas}", file=sys.stderr, flush=True)
    ms, _ = time_steps(run, probes, args.steps, args.warmup, queue_ahead=True)
    _, kms = time_steps(run, probes, args.steps, 0, queue_ahead=True, per_kernel=True)
    ms_host, _ = time_steps(run, probes, args.steps, 0, queue_ahead=False)
    ms_warm, _ = time_steps(run, probes, args.steps, 2, queue_ahead=True, warm=True)
    keys = wl.visible_keys
    work = run.score_work()
    scale = 1e9 if work["unit"] == "GB/s" else 1e12
    achieved = work["work"] / (kms["score"] / 1e3) / scale
    measured_peak = peaks.get(work["peak_key"]) if peaks else None
    st_work = run.score_topk_work()
    st_ms = kms["score"] + kms["topk"]
    st_achieved = st_work / (st_ms / 1e3) / scale
    entry = {
        "workload": name,
        "description": run.desc,
        "ms_per_step": ms,
        "ms_per_step_host_paced": ms_host,
        "ms_per_step_warm": ms_warm,
        "keys_per_s": keys / (ms / 1e3),
        "selections_per_s": wl.rows / (ms / 1e3),
        "selected_indices_per_s": float(np.minimum(wl.row_len, wl.k).sum()) / (ms / 1e3),
        "kernel_ms": kms,
        "config": {"rows": wl.rows, "visible_keys": keys, "max_row_len": wl.max_row_len, "k": wl.k,
                   "heads": wl.heads, "head_dim": 128, "key_dtype": run.kd, "q_dtype": wl.q_dtype,
                   "block_size": wl.block_size, "new_tokens_stored_per_step": int(wl.new_x_bits.shape[0]),
                   "cache_replicas": run.replicas},
        "roofline": {
            "bound": work["bound"], "kernel": work["kernel"], "achieved": achieved, "peak": work["peak"],
            "unit": work["unit"], "frac": achieved / work["peak"],
            "frac_of_measured_peak": (achieved / measured_peak) if measured_peak else None,
            "traffic": traffic_from_profile(work["kernel"], name),
            "algorithmic_per_launch": work["work"], "algorithmic_per_unit": work["per_unit"],
            "time": ("mean score-kernel interval between fence-free HIP events on the launch stream, "
                     "steps queued ahead"),
        },
        "score_topk_roofline": {
            "bound": work["bound"], "achieved": st_achieved, "peak": work["peak"], "unit": work["unit"],
            "frac": st_achieved / work["peak"],
            "frac_of_measured_peak": (st_achieved / measured_peak) if measured_peak else None,
            "algorithmic_per_step": st_work, "ms": st_ms,
            "work": ("keys + table + q + w + selected indices (no intermediate scores)" if not run.prefill
                     else "16,384 FLOP per visible pair, over the score and top-k kernels' time"),
        },
    }
    if not args.no_cpu_baseline:
        entry["cpu_baseline"] = cpu_baseline(wl, run.kd, cpu_budget or args.cpu_budget)
    del run
    torch.cuda.empty_cache()
    return entry


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--per-config", default=",".join(PER_CONFIG),
                    help="comma-separated workloads measured after the headline (default: the other "
                         "configurations); empty for none")
    ap.add_argument("--no-per-config", action="store_true", help="only the headline workload")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak kernels")
    ap.add_argument("--replicas", type=int, default=None, help="key-cache replicas (default: cold-cache rotation)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time, headline")
    ap.add_argument("--cpu-budget-per-config", type=float, default=6.0)
    ap.add_argument("--op", default="step", choices=["step", "q_prep", "translate", "attention"],
                    help="step: the indexer step (default); q_prep: the query preparation alone, on "
                         "the workload's queries; translate: logical -> physical translation of "
                         "top-k-shaped selections, and what the fused slots add to score + top-k; "
                         "attention: sparse attention over 32 rows x top-512 slots")
    ap.add_argument("--heads", type=int, default=16, help="query heads of --op attention")
    ap.add_argument("--no-attention", action="store_true", help="skip the sparse-attention block")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the indexer path runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    if "RANK" in os.environ and os.environ.get("WORLD_SIZE", "1") != "1":
        print("single-GPU benchmark: run without torch.distributed", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    probes = Probes()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {n} bytes read, {n} bytes written", file=sys.stderr, flush=True)
        del src, dst

    if args.op in ("q_prep", "translate"):
        run = Runner(args.workload, args.replicas)
        fn = bench_q_prep if args.op == "q_prep" else bench_translate
        print(json.dumps(fn(args, run)), flush=True)
        return
    if args.op == "attention":
        res = bench_attention(probes, args.steps, args.warmup, args.heads)
        print(json.dumps({"metric": "sparse-attention rows/s over top-k selected KV slots at 1 GPU",
                          "value": res["rows_per_s"], "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": res["ms_per_launch"], "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": res["workload"], "parallelism": "single GPU"}, **res}),
              flush=True)
        return

    peaks = None if args.no_peaks else probes.peaks()
    if peaks:
        print(f"[bench] measured peaks: {json.dumps(peaks)}", file=sys.stderr, flush=True)
    head = measure(args.workload, args, probes, peaks)
    cfg = head["config"]
    line = {
        "metric": METRIC,
        "value": head["keys_per_s"],
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if cfg["q_dtype"] == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": head["description"], **cfg,
                   "parallelism": "single GPU"},
        "selections_per_s": head["selections_per_s"],
        "selected_indices_per_s": head["selected_indices_per_s"],
        "ms_per_step_host_paced": head["ms_per_step_host_paced"],
        "ms_per_step_warm": head["ms_per_step_warm"],
        "kernel_ms": head["kernel_ms"],
        "roofline": head["roofline"],
        "score_topk_roofline": head["score_topk_roofline"],
        "timing": ("steps queued behind a device-side delay and run back to back; HIP events on the "
                   "launch stream bracket the region and each kernel; ms_per_step_host_paced is the "
                   "same loop launched at the host's own pace; ms_per_step_warm reads one key-cache "
                   "replica every step (cache-resident where it fits) instead of rotating replicas"),
        "peaks_measured": peaks,
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if not args.no_per_config and args.per_config:
        from synth import gen
        cache = {}
        per = {}
        for name in [n for n in args.per_config.split(",") if n and n != args.workload]:
            cfgi, kd, _ = WORKLOADS[name]
            if cfgi not in cache:        # the A/B pair shares one set of keys
                cache = {cfgi: gen.config(cfgi, key_dtype=kd)}
            wl = cache[cfgi]
            wl.key_dtype = kd
            per[name] = measure(name, args, probes, peaks, wl=wl, cpu_budget=args.cpu_budget_per_config)
        line["per_config"] = per
    if not args.no_attention:    # the consumer of the selections, at the decode-batch shape
        line["sparse_attention"] = {f"heads_{h}": bench_attention(probes, max(args.steps, 20), args.warmup, h)
                                    for h in (16, 64)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
