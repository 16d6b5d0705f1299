#!/usr/bin/env python3
"""Benchmark of the DSA indexer hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input, with every
input already resident in HBM:
  decode workloads   index_k_store of the step's new tokens (RMSNorm -> RoPE ->
                     Hadamard -> fp8 -> paged scatter), indexer_score over the
                     paged cache, indexer_topk of every row
  prefill workload   indexer_quant_fp8 of the queries, indexer_score (fp8 x fp8),
                     indexer_topk
These are exactly the kernels indexer_score_topk chains; calling the three entry
points separately lets HIP events on the launch stream time each kernel inside the
timed region.  Key caches are replicated and rotated so that every step reads its
keys from HBM, not from the 256 MB last-level cache.

Prints one JSON line.  Metric: visible (query, key) pairs scored per second for the
whole step, with top-k selections per second beside it; `roofline` reports the
dominant kernel against the HBM (decode) or fp8 MFMA (prefill) peak.
"""
from __future__ import annotations

import argparse
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
COLD_BYTES = 640 << 20          # replicas of the key cache cover at least this much

WORKLOADS = {
    # name: (config, key dtype, description)
    "decode_b32": (2, "fp8", "decode batch 32, S~U[4500,22000], fp8 keys, top-512"),
    "tiny_decode": (1, "bf16", "decode 1 x 2000, bf16 keys, top-512"),
    "ab_bf16": (3, "bf16", "decode 16 x 131072, bf16 keys, top-1024"),
    "ab_fp8": (3, "fp8", "decode 16 x 131072, fp8 keys, top-1024"),
    "ab_fp4": (3, "fp4", "decode 16 x 131072, MXFP4 keys (e2m1 + e8m0 per 32), top-1024"),
    "prefill": (4, "fp8", "chunked prefill 4096 rows on a 32768 prefix, fp8 keys, top-1024"),
    "prefill_fp4": (4, "fp4", "chunked prefill 4096 rows on a 32768 prefix, MXFP4 keys, top-1024"),
    "long_decode": (5, "fp8", "decode 4 x 1048576 fp8 keys after a 4096-token store, top-1024"),
}


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_attention_token_store_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"score_decode": ["score_decode.hip", "common.hpp"],
                  "score_prefill": ["score_prefill.hip", "common.hpp"],
                  "q_prep": ["store.hip", "common.hpp"],
                  "translate": ["topk.hip", "common.hpp"]}


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


class Runner:
    def __init__(self, name: str, replicas: int | None):
        import torch
        import sparse_attention_token_store_amd as dsa
        from synth import gen
        self.torch, self.dsa, self.name = torch, dsa, name
        cfg, kd, self.desc = WORKLOADS[name]
        wl = gen.config(cfg, key_dtype=kd)
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
        recorded around the score kernel and the top-k."""
        dsa, wl = self.dsa, self.wl
        cache = self.caches[i % self.replicas]
        if wl.new_x_bits.shape[0]:
            dsa.index_k_store(self.new_x, self.new_pos, self.new_slots, cache, dsa.IDX_STORE_ALL,
                              wl.rms_eps, wl.rope_base, wl.rope_dim)
        if self.prefill:
            dsa.indexer_quant_fp8(self.q, self.q_codes, self.q_scale)
        if ev:
            ev[0].record()
        if self.prefill:
            dsa.indexer_score(self.q_codes, self.w, cache, self.rows, self.scores, q_scale=self.q_scale)
        else:
            dsa.indexer_score(self.q, self.w, cache, self.rows, self.scores)
        if ev:
            ev[1].record()
        dsa.indexer_topk(self.scores, self.row_len, wl.max_row_len, wl.k, self.out_idx, self.ws)
        if ev:
            ev[2].record()

    # algorithmic work of the dominant (score) kernel per launch
    def score_work(self):
        wl = self.wl
        keys = wl.visible_keys
        if self.prefill:
            flops = 2.0 * wl.heads * 128 * keys
            return {"bound": "mfma", "unit": "TFLOP/s", "work": flops, "peak": FP8_MFMA_PEAK_TFLOPS,
                    "kernel": "score_prefill"}
        key_bytes = {"fp8": 132, "fp4": 68, "bf16": 256}[self.kd]
        per_key = key_bytes + 4 + 4.0 / wl.block_size          # key, score write, table entry
        per_row = wl.heads * 128 * 2 + wl.heads * 4 + 8         # q (bf16), w, row_seq + row_len
        pad = sum(wl.max_row_len - int(n) for n in wl.row_len) * 4   # -inf padding writes
        nbytes = keys * per_key + wl.rows * per_row + pad
        return {"bound": "hbm", "unit": "GB/s", "work": nbytes, "peak": HBM_PEAK_GBS,
                "kernel": "score_decode"}


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


def cpu_baseline(wl, kd, budget_s=15.0, min_s=10.0):
    """The oracle (numpy float64, BLAS threads as configured) on a bounded sample of
    the same workload: whole rows (store chain of the row's new tokens, key
    dequantisation, score, top-k), repeated over the rows until about budget_s of
    CPU work (at least min_s) has been timed."""
    from oracle import oracle as O
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = None
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
                    parts.append(y)
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
    return {"value": keys_done / t_total, "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_done} rows ({keys_done} visible keys; {passes} pass(es) over the "
                      f"{wl.rows} rows of the same workload), {t_total:.1f} s: store chain of the "
                      f"row's new tokens, fp8/bf16 key decode, float64 score, sort-based top-k",
            "selections_per_s": rows_done / t_total}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b32", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=None, help="key-cache replicas (default: cold-cache rotation)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--event-every", type=int, default=8,
                    help="record the per-kernel timing events on every N-th timed step (each record is a "
                         "host call; on the short decode steps recording them every step would leave the "
                         "GPU waiting on the host)")
    ap.add_argument("--op", default="step", choices=["step", "q_prep", "translate"],
                    help="step: the indexer step (default); q_prep: the query preparation alone, on "
                         "the workload's queries; translate: logical -> physical translation of "
                         "top-k-shaped selections, and what the fused slots add to score + top-k")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    if "RANK" in os.environ and os.environ.get("WORLD_SIZE", "1") != "1":
        print("single-GPU benchmark: run without torch.distributed", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    run = Runner(args.workload, args.replicas)
    wl = run.wl
    print(f"[bench] {args.workload}: {run.desc}; rows={wl.rows} visible_keys={wl.visible_keys} "
          f"replicas={run.replicas}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {n} bytes read, {n} bytes written", file=sys.stderr, flush=True)

    if args.op == "q_prep":
        print(json.dumps(bench_q_prep(args, run)), flush=True)
        return
    if args.op == "translate":
        print(json.dumps(bench_translate(args, run)), flush=True)
        return

    for i in range(args.warmup):
        run.step(i)
    torch.cuda.synchronize()

    every = max(1, args.event_every)
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in range(0, args.steps, every)}
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        run.step(i, evs.get(i))
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / args.steps
    # kernel durations from the events of the sampled steps of this same timed region
    score_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs.values()]))
    topk_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs.values()]))

    keys = wl.visible_keys
    value = keys / (ms / 1e3)
    work = run.score_work()
    achieved = work["work"] / (score_ms / 1e3) / (1e9 if work["unit"] == "GB/s" else 1e12)
    traffic = traffic_from_profile(work["kernel"], args.workload)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if run.prefill else "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "description": run.desc,
            "rows": wl.rows,
            "visible_keys": keys,
            "max_row_len": wl.max_row_len,
            "k": wl.k,
            "heads": wl.heads,
            "head_dim": 128,
            "key_dtype": run.kd,
            "q_dtype": wl.q_dtype,
            "block_size": wl.block_size,
            "new_tokens_stored_per_step": int(wl.new_x_bits.shape[0]),
            "cache_replicas": run.replicas,
            "parallelism": "single GPU",
        },
        "selections_per_s": wl.rows / (ms / 1e3),
        "kernel_ms": {"score": score_ms, "topk": topk_ms, "sampled_steps": len(evs)},
        "roofline": {
            "bound": work["bound"],
            "kernel": work["kernel"],
            "achieved": achieved,
            "peak": work["peak"],
            "unit": work["unit"],
            "frac": achieved / work["peak"],
            "traffic": traffic,
            "algorithmic_per_launch": work["work"],
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, run.kd, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
