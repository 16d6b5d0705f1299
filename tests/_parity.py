"""The oracle's view of a workload, and the comparisons between the HIP path and
the oracle.

Comparison rules:
  scores     |g - o| <= rtol * max(|o|, 0.01 * max_p |o[r, p]|) for p < row_len and
             g == -inf exactly for row_len <= p < max_row_len.  rtol = 1e-3 for bf16
             keys, 2e-3 for fp8 keys.  The 1%-of-row-max floor keeps the test
             meaningful where a score approaches zero (every head's logit <= 0).
  selections the selected sets agree exactly outside the ambiguous positions: those
             whose oracle score o_p lies within the score tolerance of the oracle's
             k-th score tau, |o_p - tau| <= rtol * max(|tau|, 0.01 * max_p |o|), and
             store-chain keys whose fp8 code is ambiguous (below).  Sizes match;
             when k >= row_len both are every position.  (A path whose scores used
             the whole tolerance would need twice this band, since both o_p and tau
             move; the kernels' measured score error is ~1e-6 relative, far inside
             half of it.)
  store-chain codes: the HIP path quantises float32 pre-quantisation rows, the
             oracle float64 ones.  Where y/s lies within 448 * 2e-6 (the float32
             chain's error bound relative to the row absmax) of an e4m3 rounding
             midpoint, either neighbouring code is a correct rounding, so such codes
             may differ by one step; everything else is exact.  Scores of such keys
             get the tolerance widened by the most a one-step flip can move them.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O

RTOL = {"bf16": 1e-3, "fp8": 2e-3, "fp4": 2e-3}
# bound on |float32 chain - float64 chain| relative to the row's absmax (the
# float32 pipeline measures ~4e-7; the store test asserts 1e-5)
CHAIN_REL_ERR = 2e-6


def _e4m3_table():
    return O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def ambiguous_codes(y64: np.ndarray, rel=CHAIN_REL_ERR) -> np.ndarray:
    """[n,128] bool: elements of float64 pre-quantisation rows whose scaled value
    y/s lies within 448*rel of an e4m3 rounding midpoint (a float32 pipeline may
    round them either way)."""
    return _code_flip_step(y64, rel) > 0


def _code_flip_step(y64, rel):
    """[n,128] float64: for elements whose code may flip, the value gap between the
    two candidate codes (in the y/s domain); 0 elsewhere."""
    amax = np.abs(y64).max(axis=1, keepdims=True)
    s = np.where(amax < 2.0 ** -100, 1.0, amax / 448.0)
    t = np.abs(y64 / s)
    tab = _e4m3_table()
    mids = (tab[:-1] + tab[1:]) / 2
    i = np.clip(np.searchsorted(mids, t), 0, mids.size - 1)
    j = np.clip(i - 1, 0, mids.size - 1)
    di, dj = np.abs(t - mids[i]), np.abs(t - mids[j])
    k = np.where(di <= dj, i, j)
    near = np.minimum(di, dj) <= 448.0 * rel
    return np.where(near, tab[k + 1] - tab[k], 0.0)


def _bf16_flip_step(y64, rel):
    """Same for a bf16 store: the bf16 spacing where the rounding may flip."""
    amax = np.abs(y64).max(axis=1, keepdims=True)
    y32 = np.abs(y64).astype(np.float32)
    u = y32.view(np.uint32) & np.uint32(0xFFFF0000)
    lo = u.view(np.float32).astype(np.float64)
    hi = (u + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    near = np.abs(np.abs(y64) - mid) <= rel * amax
    return np.where(near, hi - lo, 0.0)


def round_bf16(y64: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (through float32, as the float32 pipeline
    rounds), as float64."""
    return O.bf16_bits_to_f64(O.bf16_round(np.asarray(y64, dtype=np.float32)))


class OracleKeys:
    """float64 keys per sequence as the oracle defines them.  For keys written by the
    store chain it also keeps, per element, the value gap to the other rounding the
    float32 pipeline may legitimately take (0 where the rounding is unambiguous)."""

    def __init__(self, wl, key_dtype=None):
        self.wl = wl
        self.key_dtype = key_dtype or wl.key_dtype
        self._new, self._gap = {}, {}
        if wl.new_x_bits.shape[0]:
            y = O.store_chain(wl.new_x_bits, wl.new_pos, O.STORE_RMSNORM | O.STORE_ROPE | O.STORE_HADAMARD,
                              wl.rms_eps, wl.rope_base, wl.rope_dim)
            if self.key_dtype == "fp8":
                codes, sc = O.quant_fp8(y.astype(np.float32))
                k = O.dequant_fp8(codes, sc)
                gap = _code_flip_step(y, CHAIN_REL_ERR) * sc.astype(np.float64)[:, None]
            else:
                k = round_bf16(y)
                gap = _bf16_flip_step(y, CHAIN_REL_ERR)
            for b in np.unique(wl.new_seq):
                sel = wl.new_seq == b
                self._new[int(b)] = k[sel]
                self._gap[int(b)] = (wl.new_pos[sel].astype(np.int64), gap[sel])

    def prefix(self, b: int, p0: int, p1: int) -> np.ndarray:
        x = self.wl.keys_bits[b][p0:p1]
        if self.key_dtype == "bf16":
            return O.bf16_bits_to_f64(x)
        if self.key_dtype == "fp4":
            return O.dequant_mxfp4(*O.quant_mxfp4(O.bf16_bits_to_f32(x)))
        return O.dequant_fp8(*O.quant_fp8(O.bf16_bits_to_f32(x)))

    def __call__(self, b: int, p0: int, p1: int) -> np.ndarray:
        n0 = int(self.wl.stored_len[b])
        parts = []
        if p0 < n0:
            parts.append(self.prefix(b, p0, min(p1, n0)))
        if p1 > n0:
            nk = self._new[b]
            parts.append(nk[max(p0, n0) - n0:p1 - n0])
        return np.concatenate(parts, 0)

    def slack(self, rows=None) -> dict:
        """{row: {position: bound}}: how far one-step rounding flips of ambiguous
        store-chain elements can move that row's score of that key:
        sum_h |w_h| sum_d |q_hd| * gap_d."""
        wl = self.wl
        rows = range(wl.rows) if rows is None else rows
        out = {}
        for i, r in enumerate(rows):
            b = int(wl.row_seq[r])
            if b not in self._gap:
                continue
            pos, gap = self._gap[b]
            hit = gap.any(axis=1)
            if not hit.any():
                continue
            q = np.abs(O.bf16_bits_to_f64(wl.q_bits[r]))          # [H,128]
            wq = np.abs(wl.w[r].astype(np.float64)) @ q            # [128]
            bounds = gap[hit] @ wq
            out[i] = {int(p): float(v) for p, v in zip(pos[hit], bounds) if p < wl.row_len[r]}
        return out


def oracle_scores(wl, okeys: OracleKeys, rows=None, q64=None) -> np.ndarray:
    """float64 [len(rows), max_row_len] scores (-inf masked).  q64: optional float64
    queries [rows, H, 128] (default: the workload's bf16 q decoded)."""
    rows = np.arange(wl.rows) if rows is None else np.asarray(rows)
    q = O.bf16_bits_to_f64(wl.q_bits[rows]) if q64 is None else q64
    return O.score_rows(q, wl.w[rows].astype(np.float64), okeys, wl.row_seq[rows], wl.row_len[rows],
                        wl.max_row_len)


def check_scores(g: np.ndarray, o: np.ndarray, row_len, rtol: float, slack=None) -> dict:
    """C1; returns stats.  slack: optional {row: {position: extra}} widening the
    tolerance of store-chain keys by their rounding-flip bound."""
    worst = 0.0
    for r in range(o.shape[0]):
        n = int(row_len[r])
        gr, orr = g[r, :o.shape[1]].astype(np.float64), o[r]
        assert np.all(np.isneginf(gr[n:])), f"row {r}: masked positions must be -inf"
        if n == 0:
            continue
        vis_g, vis_o = gr[:n], orr[:n]
        assert np.all(np.isfinite(vis_g)), f"row {r}: non-finite visible score"
        floor = 0.01 * np.max(np.abs(vis_o))
        tol = rtol * np.maximum(np.abs(vis_o), floor)
        if slack and r in slack:
            for p, v in slack[r].items():
                tol[p] += v
        err = np.abs(vis_g - vis_o)
        ok = err <= tol
        bad = np.nonzero(~ok)[0]
        assert bad.size == 0, (f"row {r}: {bad.size} scores out of tolerance, first at p={bad[0]}: "
                               f"gpu={vis_g[bad[0]]!r} oracle={vis_o[bad[0]]!r} tol={tol[bad[0]]!r}")
        worst = max(worst, float(np.max(err / np.maximum(tol, 1e-300))))
    return {"worst_err_over_tol": worst}


def check_selection(G: np.ndarray, o: np.ndarray, row_len, k: int, rtol: float, slack=None) -> dict:
    """C2 for selections G [rows, k] against oracle scores o [rows, >= max len].
    Ambiguous: |o_p - tau| <= T_tau with T_tau = rtol*max(|tau|, floor), widened by
    the store-chain slack of p and of the keys scoring tau."""
    total_amb = total_diff = 0
    for r in range(G.shape[0]):
        n = int(row_len[r])
        g = G[r]
        m = min(k, n)
        assert np.all(g[m:] == -1), f"row {r}: padding must be -1"
        gs = g[:m]
        assert np.all(np.diff(gs) > 0), f"row {r}: selection must be strictly ascending"
        assert np.all((gs >= 0) & (gs < n)), f"row {r}: selected position out of range"
        if k >= n:
            assert np.array_equal(gs, np.arange(n)), f"row {r}: k >= row_len must select every position"
            continue
        orow = o[r, :n]
        tau = O.kth_score(orow, n, k)
        floor = 0.01 * np.max(np.abs(orow))
        t_tau = rtol * max(abs(tau), floor)
        sp = np.zeros(n)
        if slack and r in slack:
            for p, v in slack[r].items():
                sp[p] += v
        s_tau = float(np.max(sp[np.abs(orow - tau) <= t_tau], initial=0.0))
        amb = np.abs(orow - tau) <= t_tau + sp + s_tau
        osel = O.topk(orow[None], [n], k)[0][:m]
        gset, oset = set(gs.tolist()), set(osel.tolist())
        ambset = set(np.nonzero(amb)[0].tolist())
        assert gset - ambset == oset - ambset, (
            f"row {r}: selections differ outside the ambiguous band: "
            f"gpu-only {sorted((gset - oset) - ambset)[:8]} oracle-only {sorted((oset - gset) - ambset)[:8]}")
        total_amb += len(ambset)
        total_diff += len(gset ^ oset)
    return {"ambiguous": total_amb, "sym_diff": total_diff}
