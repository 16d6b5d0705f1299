"""Seeded synthetic inputs shaped like the pages' indexer workloads.

Shared by the CPU oracle tests, the GPU parity tests and the benchmark.  This module
draws random numbers and lays them out; it computes none of the indexer's arithmetic
(no scoring, quantisation, normalisation, rotation or selection).

Key distribution: a Gaussian mixture (256 centres ~ N(0,1)^128, per-key noise with
sd 0.3), q ~ N(0,1), head weights w ~ U(0,1)/8, with one "needle" key per sequence
set to 4x the RMS-normalised weighted query sum.  This mirrors the planted needle of
"The Hypothesis That Refused to Die" ("Message 12994: The Synthetic Test"), a key
pointing along the weighted query and several times longer than a filler key.
Draw order from PCG64(seed) is fixed: centres, per-sequence centre indices then noise, q, w,
needle depths, page-table permutation, then hidden states of newly stored tokens.
Variable sequence lengths come from their own stream, PCG64(seed + 1).  Values are
drawn in fp32 and rounded to bf16 (round to nearest even).

Workloads (one GPU each):
  1 tiny decode     1 row, S=2000, bf16 keys, needle at 1100, top-512
  2 decode b32      32 rows, S ~ U{4500..22000}, fp8 keys, needle at 40-60%, top-512;
                    the newest key of every sequence is stored by the full store
                    chain inside the timed step
  3 A/B b16         16 rows, S=131072, the same keys as bf16 and as fp8, top-1024
  4 chunked prefill 4096 query rows on one sequence, row i sees 32768+i+1 keys,
                    fp8 keys, bf16 queries, top-1024
  5 long decode b4  4 rows, S=1048576, fp8 keys, top-1024; the last 1024 keys of
                    each sequence (4096 tokens) come from the full store chain
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 128
HEADS = 64
N_CENTRES = 256
NOISE_SD = 0.3


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even) and return the uint16 bit patterns.
    Input values are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    key_dtype: str                 # "bf16" or "fp8"
    k: int
    block_size: int
    seq_len: np.ndarray            # [B] keys per sequence (final length)
    stored_len: np.ndarray         # [B] keys written before the step (prefix)
    keys_bits: list                # per sequence: uint16 [stored_len_b, 128] bf16 keys
    needle_pos: np.ndarray         # [B] needle position per sequence (-1: none)
    q_bits: np.ndarray             # uint16 [rows, H, 128]
    w: np.ndarray                  # float32 [rows, H]
    row_seq: np.ndarray            # int32 [rows]
    row_len: np.ndarray            # int32 [rows]
    block_table: np.ndarray        # int32 [B, max_blocks]
    num_blocks: int                # physical blocks in the pool
    # tokens written by the full store chain inside the step
    new_x_bits: np.ndarray         # uint16 [n_new, 128] hidden states
    new_seq: np.ndarray            # int32 [n_new]
    new_pos: np.ndarray            # int32 [n_new]
    rope_base: float = 10000.0
    rope_dim: int = 64
    rms_eps: float = 1e-6
    q_dtype: str = "bf16"          # "bf16"; "fp8" = quantise q per (row, head) first

    @property
    def rows(self) -> int:
        return int(self.row_len.shape[0])

    @property
    def heads(self) -> int:
        return int(self.q_bits.shape[1])

    @property
    def max_row_len(self) -> int:
        return int(self.row_len.max()) if self.rows else 0

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def slots(self, seq: np.ndarray, pos: np.ndarray) -> np.ndarray:
        """Physical cache slot of (sequence, position) pairs: block * bs + offset."""
        seq = np.asarray(seq, dtype=np.int64)
        pos = np.asarray(pos, dtype=np.int64)
        blk = self.block_table[seq, pos // self.block_size].astype(np.int64)
        return blk * self.block_size + pos % self.block_size

    def prefix_tokens(self):
        """All keys stored before the step: (bf16 bits [n,128], slot [n] int64),
        concatenated over sequences in order."""
        xs, sl = [], []
        for b, kb in enumerate(self.keys_bits):
            n = kb.shape[0]
            xs.append(kb)
            sl.append(self.slots(np.full(n, b), np.arange(n)))
        return np.concatenate(xs, 0), np.concatenate(sl, 0)

    def new_slots(self) -> np.ndarray:
        return self.slots(self.new_seq, self.new_pos)

    @property
    def visible_keys(self) -> int:
        return int(self.row_len.astype(np.int64).sum())


def _page_table(rng, seq_len, bs, shuffle):
    nblk = [(int(n) + bs - 1) // bs for n in seq_len]
    pool = int(sum(nblk))
    phys = rng.permutation(pool).astype(np.int32) if shuffle else np.arange(pool, dtype=np.int32)
    table = np.zeros((len(seq_len), max(nblk) if nblk else 1), dtype=np.int32)
    off = 0
    for b, m in enumerate(nblk):
        table[b, :m] = phys[off:off + m]
        off += m
    return table, pool


def _needle(q_bits_row, w_row):
    """4 * sqrt(128) * v / ||v|| with v = sum_h w_h q_h: a key along the weighted
    query direction with per-element RMS 4 (four times a filler key's ~1)."""
    q = bf16_bits_to_f32(q_bits_row).astype(np.float64)
    v = (np.asarray(w_row, dtype=np.float64)[:, None] * q).sum(0)
    return f32_to_bf16_bits((4.0 * math.sqrt(HEAD_DIM) * v / np.linalg.norm(v)).astype(np.float32))


def make(seq_len, *, rows_per_seq=None, key_dtype="fp8", k=512, block_size=64, shuffle=True,
         needle_depth=(0.4, 0.6), needle_at=None, n_new_per_seq=0, prefill_rows=0,
         heads=HEADS, seed=0, name="custom", q_dtype="bf16", rope_base=10000.0,
         rope_dim=64, rms_eps=1e-6) -> Workload:
    """General generator.

    seq_len: keys per sequence.  Decode layout (default): one query row per sequence
    that sees every key.  Prefill layout (prefill_rows = m > 0, single sequence): m
    query rows, row i sees seq_len - m + i + 1 keys.  n_new_per_seq > 0 leaves the
    last n keys of each sequence to the store chain (hidden states drawn here).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_len = np.asarray(seq_len, dtype=np.int64)
    B = seq_len.shape[0]
    centres = rng.standard_normal((N_CENTRES, HEAD_DIM), dtype=np.float32)
    stored = seq_len - n_new_per_seq
    keys = []
    for b in range(B):
        n = int(stored[b])
        idx = rng.integers(0, N_CENTRES, size=n)
        noise = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
        keys.append(f32_to_bf16_bits(centres[idx] + np.float32(NOISE_SD) * noise))
    if prefill_rows:
        assert B == 1
        rows = prefill_rows
        row_seq = np.zeros(rows, dtype=np.int32)
        row_len = (seq_len[0] - prefill_rows + np.arange(rows) + 1).astype(np.int32)
    else:
        rows = B
        row_seq = np.arange(B, dtype=np.int32)
        row_len = seq_len.astype(np.int32)
    q_bits = f32_to_bf16_bits(rng.standard_normal((rows, heads, HEAD_DIM), dtype=np.float32))
    w = (rng.random((rows, heads), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    needle_pos = np.full(B, -1, dtype=np.int64)
    if needle_at is not None or needle_depth is not None:
        depths = rng.uniform(needle_depth[0], needle_depth[1], size=B) if needle_depth else None
        for b in range(B):
            p = int(needle_at) if needle_at is not None else int(depths[b] * int(stored[b]))
            p = min(p, int(stored[b]) - 1)
            r = int(np.nonzero(row_seq == b)[0][0])
            keys[b][p] = _needle(q_bits[r], w[r])
            needle_pos[b] = p
    table, pool = _page_table(rng, seq_len, block_size, shuffle)
    if n_new_per_seq:
        new_x = f32_to_bf16_bits(rng.standard_normal((B * n_new_per_seq, HEAD_DIM), dtype=np.float32))
        new_seq = np.repeat(np.arange(B, dtype=np.int32), n_new_per_seq)
        new_pos = np.concatenate([np.arange(int(stored[b]), int(seq_len[b]), dtype=np.int32) for b in range(B)])
    else:
        new_x = np.zeros((0, HEAD_DIM), dtype=np.uint16)
        new_seq = np.zeros(0, dtype=np.int32)
        new_pos = np.zeros(0, dtype=np.int32)
    return Workload(name=name, key_dtype=key_dtype, k=k, block_size=block_size, seq_len=seq_len,
                    stored_len=stored, keys_bits=keys, needle_pos=needle_pos, q_bits=q_bits, w=w,
                    row_seq=row_seq, row_len=row_len, block_table=table, num_blocks=pool,
                    new_x_bits=new_x, new_seq=new_seq, new_pos=new_pos, rope_base=rope_base,
                    rope_dim=rope_dim, rms_eps=rms_eps, q_dtype=q_dtype)


CONFIG_NAMES = {
    1: "tiny decode: 1 x S=2000, bf16 keys, top-512",
    2: "decode b32: 32 x S~U[4500,22000], fp8 keys, top-512",
    3: "A/B decode b16: 16 x S=131072, bf16 and fp8 keys, top-1024",
    4: "chunked prefill: 4096 rows on a 32768 prefix, fp8 keys, top-1024",
    5: "long decode b4: 4 x S=1048576, fp8 keys, top-1024, 4096-token store",
}


def config(i: int, *, scale: float = 1.0, block_size: int = 64, seed: int = 0,
           shuffle: bool | None = None, key_dtype: str | None = None) -> Workload:
    """The five workloads.  scale < 1 shrinks sequence lengths (and prefill rows) for
    quick tests while keeping their structure."""
    def sc(n):
        return max(1, int(round(n * scale)))

    if i == 1:
        return make([sc(2000)], key_dtype=key_dtype or "bf16", k=512, block_size=block_size,
                     shuffle=bool(shuffle), needle_at=sc(1100), needle_depth=None, seed=seed,
                     name="tiny_decode")
    if i == 2:
        rng = np.random.Generator(np.random.PCG64(seed + 1))
        lens = rng.integers(sc(4500), sc(22000) + 1, size=32)
        return make(lens, key_dtype=key_dtype or "fp8", k=512, block_size=block_size,
                     shuffle=True if shuffle is None else shuffle, n_new_per_seq=1, seed=seed,
                     name="decode_b32")
    if i == 3:
        return make([sc(131072)] * 16, key_dtype=key_dtype or "fp8", k=1024, block_size=block_size,
                     shuffle=True if shuffle is None else shuffle, seed=seed, name="ab_decode_b16")
    if i == 4:
        m = sc(4096)
        return make([sc(32768) + m], key_dtype="fp8", k=1024, block_size=block_size,
                     shuffle=True if shuffle is None else shuffle, needle_depth=None,
                     prefill_rows=m, seed=seed, name="chunked_prefill", q_dtype="fp8")
    if i == 5:
        n_new = sc(1024)
        return make([sc(1048576)] * 4, key_dtype="fp8", k=1024, block_size=block_size,
                     shuffle=True if shuffle is None else shuffle, needle_depth=None,
                     n_new_per_seq=n_new, seed=seed, name="long_decode_b4")
    raise ValueError(i)


def score_rows_for_topk(rows: int, n: int, *, kind: str = "normal", seed: int = 0) -> np.ndarray:
    """Synthetic fp32 score rows [rows, n] for exercising a top-k on its own.

    kinds: normal (continuous), ties (few distinct values, many ties), equal (one
    value), increasing, decreasing, signed_zero (mix of +0, -0 and positives),
    heavy (scores shaped like ReLU-weighted head sums: many exact zeros and a long
    positive tail)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "normal":
        x = rng.standard_normal((rows, n), dtype=np.float32) * np.float32(7.0)
    elif kind == "ties":
        x = rng.integers(-8, 9, size=(rows, n)).astype(np.float32) * np.float32(0.25)
    elif kind == "equal":
        x = np.full((rows, n), 1.5, dtype=np.float32)
    elif kind == "increasing":
        x = np.tile(np.arange(n, dtype=np.float32), (rows, 1))
    elif kind == "decreasing":
        x = np.tile(-np.arange(n, dtype=np.float32), (rows, 1))
    elif kind == "signed_zero":
        x = rng.integers(0, 3, size=(rows, n)).astype(np.float32)
        neg = rng.random((rows, n)) < 0.5
        x = np.where((x == 0) & neg, np.float32(-0.0), x).astype(np.float32)
    elif kind == "heavy":
        g = rng.standard_normal((rows, n), dtype=np.float32)
        x = np.maximum(g, 0).astype(np.float32) ** 3
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------------
# Inputs of the sparse attention over the selections: query heads and one 512-dim
# compressed KV state per token slot (drawn, not derived: the pages give neither).
# ----------------------------------------------------------------------------------

KV_DIM = 512


def kv_states(num_slots: int, *, seed: int = 0, sd: float = 1.0) -> np.ndarray:
    """bf16 bits [num_slots, 512]: N(0, sd^2) per element (own stream, PCG64(seed + 7))."""
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    return f32_to_bf16_bits((rng.standard_normal((num_slots, KV_DIM), dtype=np.float32) * np.float32(sd)))


def attention_case(rows: int, heads: int, k: int, num_slots: int, *, pad_frac: float = 0.0,
                   seed: int = 0, q_sd: float = 1.0):
    """Query heads (bf16 bits [rows, heads, 512], N(0, q_sd^2)) and slot lists (int64
    [rows, k]: distinct slots per row, min(k, num_slots) of them, drawn from
    [0, num_slots); a fraction pad_frac of the entries set to -1 padding, -1 also past
    num_slots)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = f32_to_bf16_bits(rng.standard_normal((rows, heads, KV_DIM), dtype=np.float32) * np.float32(q_sd))
    slots = np.full((rows, k), -1, dtype=np.int64)
    for r in range(rows):
        m = min(k, num_slots)
        slots[r, :m] = rng.choice(num_slots, m, replace=False)
    if pad_frac > 0:
        slots[rng.random((rows, k)) < pad_frac] = -1
    return q, slots
