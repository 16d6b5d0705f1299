"""CPU oracle for the DSA lightning-indexer hot path (TEST INFRASTRUCTURE ONLY).

This module is the slow, plain, obviously-correct definition that the HIP path is
checked against.  Only the test suite, the smoke check and the CPU-baseline leg of
the benchmark may import it; the product library never does, and it shares no
code, tables or constants with the HIP sources.

Everything floating point is computed in float64 on exactly-decoded inputs, except
the fp8 quantiser, whose output is a set of integer codes and is therefore specified
in float32 (see ``quant_fp8``).

Sources (web pages; cited by title and section):
  [ATOM-1507]  "[DeepSeek-V4] index_topk=1024 sparse indexer can't recall verbatim
               lines from ~18k+ prompts" (ROCm/ATOM issue 1507)
  [PIVOT-DIAG] "The Pivot: Diagnosing a Sparse Attention Recall Bug at the
               Intersection of Precision and Production"
  [PIVOT-EDIT] "The Pivot: A Single Edit That Finally Fixed DeepSeek V4's
               Long-Context Recall Failure"
  [HYPOTHESIS] "The Hypothesis That Refused to Die: When Synthetic Tests
               Contradict Real-World Failure"

Readings where the pages are silent are marked READING and are the plainest ones
the rest of the pages support.

Pin status of every public function (what fixes it other than itself is in
tests/test_oracle_*.py):
  bf16_bits_to_f64, bf16_round ............ pinned (torch bfloat16 on every bit
                                             pattern and on a sample of float32)
  e4m3_decode, e4m3_encode, quant_fp8 ..... pinned (format definition values,
                                             torch float8_e4m3fn, exact rationals)
  hadamard_matrix, rmsnorm, rope,
  store_chain ............................. pinned (closed forms, invariants,
                                             scipy.linalg.hadamard)
  q_prep .................................... pinned (per-vector brute force, the
                                             rotation identities, RoPE's relative-
                                             position property)
  e2m1_decode, e2m1_encode, quant_mxfp4,
  dequant_mxfp4 ............................ pinned (OCP value table, exact-rational
                                             nearest-value brute force, the block
                                             exponent's defining inequality, error
                                             bound, a hand-worked block)
  score, score_rows ....................... pinned (exact-rational brute force,
                                             closed forms, invariants)
  topk, kth_score ........................... pinned (subset brute force, numpy and
                                             torch library routines; a hand-worked
                                             row with ties; the order-statistic
                                             counting definition)
  translate ................................ pinned (hand-worked example, the
                                             identity table's closed form, the
                                             store's slot of every stored position,
                                             injectivity on a shuffled table)
  jaccard .................................. pinned (the printed table of the
                                             synthetic fp8-vs-bf16 test)
  sparse_attention, merge_attention ....... pinned (torch's scaled-dot-product
                                             attention in float64, closed forms for
                                             one slot and for a zero query, dense
                                             attention when every slot is listed,
                                             permutation invariance, the merge
                                             identity over disjoint sets)
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
E4M3_MAX = 448.0

# ----------------------------------------------------------------------------------
# bf16 / fp32 helpers (exact conversions only)
# ----------------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value of each finite float32 (ties to the even last mantissa
    bit), as uint16 bit patterns.  The bf16 store keeps a key this way
    ([PIVOT-EDIT] "Assumptions and Input Knowledge": 256 bytes per bf16 token).

    The two candidates are the bf16 values just below and just above |x| in
    magnitude (the float32 with its low 16 bits cleared, and the next bf16 up);
    |x| is compared with their midpoint exactly in float64."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x32)):
        raise ValueError("bf16_round: finite inputs only")
    u = x32.view(np.uint32)
    sign = u & np.uint32(0x80000000)
    lo = u & np.uint32(0x7FFF0000)                       # magnitude truncated to bf16
    hi = lo + np.uint32(0x10000)                          # next bf16 magnitude up
    a = np.abs(x32.astype(np.float64))
    v_lo = lo.view(np.float32).astype(np.float64)
    v_hi = hi.view(np.float32).astype(np.float64)         # (may be +inf: then a < mid)
    mid = (v_lo + v_hi) / 2.0
    odd = ((lo >> np.uint32(16)) & np.uint32(1)) == 1
    pick_hi = (a > mid) | ((a == mid) & odd)
    mag = np.where(pick_hi, hi, lo)
    return ((mag | sign) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------------
# OCP FP8 E4M3 (e4m3fn): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
# infinities, NaN = S.1111.111.  The pages only say the index keys are "e4m3" fp8
# with three mantissa bits ([HYPOTHESIS], "Input Knowledge Required", item 3) and a
# per-token fp32 scale, 132 bytes per token ([PIVOT-EDIT], "Assumptions and Input
# Knowledge").  READING: the OCP e4m3fn flavour, which is the native fp8 of the
# target GPU; largest finite magnitude 448.
# ----------------------------------------------------------------------------------


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3fn code as float64 (NaN for 0x7F / 0xFF).

    Normal codes (exponent field e > 0): (-1)^s * 2^(e-7) * (1 + m/8).
    Subnormal codes (e == 0):            (-1)^s * 2^(-6) * (m/8).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _e4m3_positive_table() -> np.ndarray:
    """The 127 finite non-negative e4m3 values, indexed by code 0x00..0x7E."""
    return e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Round float32 values to e4m3fn codes: nearest finite value, ties to the code
    with an even mantissa (round-to-nearest-even), saturating to +-448, keeping the
    sign (so -0 and negative underflow give 0x80).

    READING (quantiser rounding): round-to-nearest-even with saturation.  Under
    absmax scaling saturation is never reached except through the all-zero rule.

    The comparison is exact: every float32 and every e4m3 midpoint is exactly
    representable in float64, and the value is compared with the midpoint of its two
    neighbouring codes rather than with a difference that could round.
    """
    x32 = np.asarray(x, dtype=np.float32)
    if np.isnan(x32).any():
        raise ValueError("e4m3_encode: NaN input")
    sign = (x32.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    a = np.abs(x32.astype(np.float64))
    table = _e4m3_positive_table()                 # ascending, codes 0..126
    hi = np.searchsorted(table, a, side="left")    # first table value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    v_lo, v_hi = table[lo], table[hi]
    mid = (v_lo + v_hi) / 2.0                      # exact (dyadic, few bits)
    exact_hit = v_hi == a
    pick_hi = (a > mid) | ((a == mid) & (hi % 2 == 0))
    code = np.where(exact_hit, hi, np.where(pick_hi, hi, lo))
    code = np.where(a >= E4M3_MAX, 126, code)      # saturate (satfinite)
    return (code.astype(np.uint8) | (sign << np.uint8(7))).astype(np.uint8)


def quant_fp8(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-vector absmax fp8 quantisation of rows of 128 values.

    The pages store each index key as 128 e4m3 codes plus one fp32 scale (132 B per
    token, [PIVOT-EDIT] "Assumptions and Input Knowledge"); write, read and scale are
    each checked with zero error ([ATOM-1507] "How it was isolated").  They do not
    print the quantiser.  READING (the plainest per-token absmax form):
        amax = max_i |x_i|                      (float32, exact)
        s    = fl32(amax / 448)                 (correctly rounded fp32 division)
        c_i  = e4m3_encode(fl32(x_i / s))       (correctly rounded fp32 division)
    and, for an all-zero (or vanishingly small, amax < 2^-100) vector, s = 1, which
    yields all-zero codes.  Dequantised value: s * decode(c_i).

    Input: float32-representable values, shape [..., 128].  Returns (codes uint8
    [..., 128], scales float32 [...]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax < np.float32(2.0 ** -100), np.float32(1.0), s).astype(np.float32)
    y = (x32 / s[..., None]).astype(np.float32)
    return e4m3_encode(y), s


def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 value of quantised vectors: scale * decode(code), exact."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


# ----------------------------------------------------------------------------------
# fp4 index keys.  The pages name an fp4 variant of the indexer key only as a call,
# fp4_act_quant_inplace(kv, 32), applied after the rotation, and as "the fp4 QAT
# round-trip" ([ATOM-1507] "Where" and "Recommended fix").  READING: OCP MXFP4, the
# microscaling format with 32-element blocks: e2m1 elements (1 sign, 2 exponent bits
# with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one e8m0
# scale 2^(E-127) per block.  The shared exponent is floor(log2(amax)) - 2 (2 being
# the largest e2m1 exponent), limited to the e8m0 range [-127, 127]; each element is
# x / 2^e rounded to the nearest e2m1 value, ties to the even mantissa, saturating at
# +-6.  An all-zero block takes the scale 2^0.  The round trip through these codes
# is the QAT round trip, so storing the codes and widening them at read time gives
# the same values.
# ----------------------------------------------------------------------------------

E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each 4-bit e2m1 code (bit 3 = sign) as float64."""
    c = np.asarray(codes, dtype=np.int64)
    mag = np.asarray(E2M1_MAGNITUDES)[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """Nearest e2m1 code of each value: ties to the code with an even mantissa bit,
    saturating at +-6, the sign kept (-0 gives code 8).  The comparison with the
    midpoint of the two neighbouring magnitudes is exact in float64."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e2m1_encode: NaN input")
    a = np.abs(v)
    table = np.asarray(E2M1_MAGNITUDES)
    hi = np.minimum(np.searchsorted(table, a, side="left"), 7)   # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    mid = (table[lo] + table[hi]) / 2.0
    pick_hi = (table[hi] == a) | (a > mid) | ((a == mid) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a > 6.0, 7, code)
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def quant_mxfp4(x, block: int = 32) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 quantisation of rows of 128 values in blocks of `block` (the reading
    above).  Returns (codes uint8 [..., 128] holding one 4-bit code each,
    e8m0 uint8 [..., 128 // block] biased exponents)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    shp = x.shape
    xb = x.reshape(shp[:-1] + (shp[-1] // block, block))
    amax = np.abs(xb).max(axis=-1)
    # floor(log2(amax)) from the exact binary exponent (np.log2 may round up just
    # below a power of two): frexp gives amax = m * 2^q with m in [0.5, 1)
    _, q = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, (q - 1) - 2, 0)
    e = np.clip(e, -127, 127)
    codes = e2m1_encode(xb / np.ldexp(1.0, e)[..., None])
    return codes.reshape(shp), (e + 127).astype(np.uint8)


def dequant_mxfp4(codes, e8m0, block: int = 32) -> np.ndarray:
    c = np.asarray(codes)
    shp = c.shape
    vals = e2m1_decode(c).reshape(shp[:-1] + (shp[-1] // block, block))
    scale = np.ldexp(1.0, np.asarray(e8m0, dtype=np.int64) - 127)
    return (vals * scale[..., None]).reshape(shp)


# ----------------------------------------------------------------------------------
# Index-K store chain: RMSNorm -> RoPE -> Hadamard -> (quantise) -> paged write.
# Order: [PIVOT-EDIT] "The Reasoning Behind the Edit" describes an unfused key path
# that normalises the key, applies its rotary embedding and rotates it, and only
# then writes it to the cache; [ATOM-1507] "Where" puts the interleaved RoPE on the
# trailing rope_dim ahead of the Walsh-Hadamard rotation.
# ----------------------------------------------------------------------------------

STORE_RMSNORM = 1
STORE_ROPE = 2
STORE_HADAMARD = 4


def hadamard_matrix(n: int = HEAD_DIM) -> np.ndarray:
    """Unnormalised Walsh-Hadamard matrix in Sylvester (natural) order, by the
    recursion H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]].  Integer entries +-1.

    [ATOM-1507] "Root cause found": H is orthogonal, so (Hq).(Hk) = q.k once it is
    normalised by 1/sqrt(n).  READING: natural (Sylvester) order.
    """
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps), unit gain, float64.

    [PIVOT-EDIT] "The Reasoning Behind the Edit" names normalisation as the first
    store step; READING: RMS normalisation with unit gain (the gain is a trained
    weight the pages do not give) and eps a parameter.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, positions: np.ndarray, base: float, rope_dim: int) -> np.ndarray:
    """Interleaved rotary embedding on the trailing rope_dim dimensions, float64.

    With o = 128 - rope_dim, pair i = (x[o+2i], x[o+2i+1]) is rotated by the angle
    theta_i = pos * base^(-2i/rope_dim):
        x'[o+2i]   = x[o+2i] cos(theta_i) - x[o+2i+1] sin(theta_i)
        x'[o+2i+1] = x[o+2i] sin(theta_i) + x[o+2i+1] cos(theta_i)
    Dimensions below o are untouched.  ([ATOM-1507] "Where": "interleaved RoPE to
    trailing rope_dim".)  The angle is formed in float64; positions reach ~1M.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    if rope_dim % 2 or not (2 <= rope_dim <= d):
        raise ValueError("rope_dim must be even and in [2, head_dim]")
    o = d - rope_dim
    i = np.arange(rope_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * i / rope_dim)            # [rope_dim/2]
    theta = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(theta), np.sin(theta)
    a = x[:, o::2].copy()
    b = x[:, o + 1::2].copy()
    x[:, o::2] = a * c - b * s
    x[:, o + 1::2] = a * s + b * c
    return x


def store_chain(x_bits: np.ndarray, positions: np.ndarray, flags: int, eps: float,
                base: float, rope_dim: int) -> np.ndarray:
    """float64 pre-quantisation rows of the index-K store: decoded bf16 input, then
    (optionally) RMSNorm, RoPE and the normalised Hadamard rotation y = H x / sqrt(128),
    in that order.  Returns float64 [n, 128]."""
    y = bf16_bits_to_f64(x_bits)
    if flags & STORE_RMSNORM:
        y = rmsnorm(y, eps)
    if flags & STORE_ROPE:
        y = rope(y, positions, base, rope_dim)
    if flags & STORE_HADAMARD:
        h = hadamard_matrix(y.shape[-1]).astype(np.float64)
        y = (y @ h.T) / np.sqrt(float(y.shape[-1]))
    return y


def q_prep(q_bits: np.ndarray, positions: np.ndarray, flags: int, base: float, rope_dim: int,
           eps: float = 1e-6) -> np.ndarray:
    """float64 query preparation: every (row, head) vector of the decoded bf16 query
    [rows, heads, 128] goes through the same chain as an index key (optional
    RMSNorm, interleaved RoPE on the trailing rope_dim at its row's position, the
    normalised Hadamard rotation), all heads of a row sharing the row's position.

    [ATOM-1507] "Where": the index query is prepared by interleaved RoPE on the
    trailing rope_dim followed by a Hadamard rotation (plus fp8 quantisation, which
    is quant_fp8 applied to these rows).  "Root cause found": the key must carry the
    same rotation, since (H q).(H k) = q.k for the orthogonal H while (H q).k is a
    scrambled product.  Returns float64 [rows, heads, 128]."""
    q_bits = np.asarray(q_bits)
    rows, heads, d = q_bits.shape
    pos = np.repeat(np.asarray(positions, dtype=np.int64).reshape(rows), heads)
    y = store_chain(q_bits.reshape(rows * heads, d), pos, flags, eps, base, rope_dim)
    return y.reshape(rows, heads, d)


# ----------------------------------------------------------------------------------
# Indexer score
# ----------------------------------------------------------------------------------


def score(q: np.ndarray, w: np.ndarray, keys: np.ndarray, row_len: int | None = None) -> np.ndarray:
    """Relevance score of every visible key for one query row, float64.

        o[p] = sum_h w[h] * max(0, sum_d q[h, d] * k[p, d])   for p < row_len

    The pages name the parts: a query-key dot product per index head ([ATOM-1507]
    "Root cause found", [HYPOTHESIS] "The Context": a compressed query-key dot
    product), a per-head weights projection and a softmax scaling ([HYPOTHESIS]
    "The Bash Command").  READING: ReLU of each head's logit, weighted by w_h and
    summed over heads; any positive global scale is folded into w (it cannot change
    a top-k since ReLU(cx) = c ReLU(x) for c > 0).  Keys at p >= row_len are never
    read (causal / committed-key mask).

    q: [H, 128], w: [H], keys: [L, 128] (already dequantised, float64).
    Returns float64 [row_len].
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n = keys.shape[0] if row_len is None else int(row_len)
    if n == 0:
        return np.zeros(0, dtype=np.float64)
    k = np.asarray(keys[:n], dtype=np.float64)
    logits = q @ k.T                                   # [H, n]
    return w @ np.maximum(logits, 0.0)                 # [n]


def score_rows(q: np.ndarray, w: np.ndarray, seq_keys, row_seq, row_len,
               max_row_len: int, chunk: int = 1 << 16) -> np.ndarray:
    """Scores of many rows laid out as a [rows, max_row_len] float64 matrix with
    -inf at masked positions (p >= row_len[r]).

    q: [rows, H, 128]; w: [rows, H]; seq_keys: sequence -> float64 keys [L_b, 128]
    (a list, or a callable taking (b, start, stop)).  Keys are consumed in chunks so
    long rows stay within memory; chunking only splits the sum over keys, not the
    sum over heads or dimensions, so it changes nothing.
    """
    rows = len(row_len)
    out = np.full((rows, max_row_len), -np.inf, dtype=np.float64)
    for r in range(rows):
        b, n = int(row_seq[r]), int(row_len[r])
        for p0 in range(0, n, chunk):
            p1 = min(n, p0 + chunk)
            k = seq_keys(b, p0, p1) if callable(seq_keys) else seq_keys[b][p0:p1]
            out[r, p0:p1] = score(q[r], w[r], k)
    return out


# ----------------------------------------------------------------------------------
# Top-k selection
# ----------------------------------------------------------------------------------


def topk(scores: np.ndarray, row_len, k: int) -> np.ndarray:
    """Causal top-k per row.

    For row r only positions p < row_len[r] are candidates.  They are ordered by
    score descending, ties broken by the lower position, and the first
    min(k, row_len[r]) are kept.  READING (output form): the kept positions are
    returned in ascending order and the row is padded with -1 to length k.  Zero
    scores of either sign compare equal (they are the same number).  READING (NaN):
    a NaN score, of either sign and any payload, ranks above every number and all
    NaNs tie, which is how torch.topk orders values.

    ([ATOM-1507] "Summary"/"How it was isolated": index_topk of 512 or 1024 kept
    per row; the selection kernel is judged by overlap with torch.topk.)
    """
    scores = np.asarray(scores)
    rows = scores.shape[0]
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        n = int(row_len[r])
        if n <= 0:
            continue
        with np.errstate(invalid="ignore"):              # (signalling-NaN inputs)
            s = scores[r, :n].astype(np.float64)
        nan = np.isnan(s)
        value = np.where(nan, 0.0, s)
        # primary key: NaN first; then score descending; then the lower position
        order = np.lexsort((np.arange(n), -value, ~nan))
        keep = np.sort(order[:min(k, n)])
        out[r, :keep.size] = keep
    return out


def kth_score(scores_row: np.ndarray, n: int, k: int) -> float:
    """The k-th largest visible score of a row (the selection threshold tau)."""
    s = np.sort(np.asarray(scores_row[:n], dtype=np.float64))[::-1]
    return float(s[min(k, n) - 1])


def rank_of(scores_row: np.ndarray, n: int, p: int) -> int:
    """1-based rank of position p under (score desc, position asc)."""
    s = np.asarray(scores_row[:n], dtype=np.float64)
    return int(np.sum(s > s[p]) + np.sum(s[:p] == s[p]) + 1)


# ----------------------------------------------------------------------------------
# Logical -> physical translation of the selections
# ----------------------------------------------------------------------------------


def translate(idx, block_table, row_seq, row_len, block_size: int, num_blocks: int,
              max_row_len: int | None = None) -> np.ndarray:
    """Physical cache slot of every selected logical key position.

    The pages name the step (csa_translate_pack, logical -> physical) and say it is
    correct for arbitrary index lists ([ATOM-1507] "How it was isolated"); they do
    not print it.  READING: the paged layout the store writes, where position t of
    sequence s sits in logical block t // bs at offset t % bs, and the block table
    names the physical block b of that logical block:
        slot = b * bs + t % bs.
    An entry that addresses no visible key maps to -1: the -1 padding of a short
    row, t outside 0 <= t < min(row_len[r], max_row_len), a row whose sequence id is
    outside the table, a logical block past the table's width, or a physical block
    id outside [0, num_blocks).

    idx [rows][k] int; block_table [num_seqs][max_blocks]; row_seq, row_len [rows].
    Returns int64 [rows][k].
    """
    idx = np.asarray(idx, dtype=np.int64)
    table = np.asarray(block_table, dtype=np.int64)
    num_seqs, max_blocks = table.shape
    rows, k = idx.shape
    out = np.full((rows, k), -1, dtype=np.int64)
    for r in range(rows):
        s = int(row_seq[r])
        n = max(int(row_len[r]), 0)
        if max_row_len is not None:
            n = min(n, int(max_row_len))
        if not 0 <= s < num_seqs:
            continue
        t = idx[r]
        lb = np.where(t >= 0, t // block_size, 0)
        ok = (t >= 0) & (t < n) & (lb < max_blocks)
        b = np.where(ok, table[s, np.minimum(lb, max_blocks - 1)], -1)
        ok &= (b >= 0) & (b < num_blocks)
        out[r] = np.where(ok, b * block_size + t % block_size, -1)
    return out


# ----------------------------------------------------------------------------------
# fp8-vs-bf16 selection overlap
# ----------------------------------------------------------------------------------


def jaccard(a, b) -> tuple[float, int]:
    """Jaccard overlap |A n B| / |A u B| of two selections and the number of
    positions of A missing from B (|A \\ B|), -1 padding ignored.

    ([HYPOTHESIS] "Message 12994: The Synthetic Test": "jacc512" and
    "lost(bf16->fp8)" columns, with A the bf16-key selection and B the fp8-key one.)
    """
    sa = {int(v) for v in np.asarray(a).ravel() if v >= 0}
    sb = {int(v) for v in np.asarray(b).ravel() if v >= 0}
    union = sa | sb
    if not union:
        return 1.0, 0
    return len(sa & sb) / len(union), len(sa - sb)


# ----------------------------------------------------------------------------------
# Sparse attention over the selections (the consumer of the top-k)
# ----------------------------------------------------------------------------------
#
# The pages place the selections' consumer beside the indexer without printing it:
# the decode attention kernel reads the rows the indexer selected, after the logical
# -> physical translation ([ATOM-1507] "How it was isolated": the decode attention
# kernel and csa_translate_pack each checked on their own; "Root cause found": a
# key the indexer drops is invisible to sparse attention while dense attention,
# which reads every row, still sees it).  The main KV cache holds one compressed
# KV state per token of head_dim 512 ([PIVOT-EDIT] "Assumptions and Input
# Knowledge": head_dim 512 for the main KV against 128 for the indexer; the
# compressor stores compressed KV states).
#
# READING: multi-query latent attention in its absorbed form, the plainest one the
# pages support: every query head attends over the same per-token 512-dim state,
# which serves as key and as value; the score is a scaled dot product and the
# softmax runs over the listed (selected) slots only.  The log-sum-exp of each
# head's scores is returned too, so that attention over two disjoint sets (the
# sparse selection and, say, a sliding window of recent tokens, the pages' two KV
# paths) merges exactly (merge_attention below).


def sparse_attention(q: np.ndarray, kv: np.ndarray, slots: np.ndarray, scale: float):
    """float64 attention of every query head over the KV rows a row lists.

    q: [rows, H, D] query heads; kv: [num_slots, D] KV states (float64, already
    decoded); slots: [rows, k] integer slot lists, negative entries are padding.
    For row r with listed slots p_1..p_n (n >= 1; repeated slots count as often as
    they are listed), and each head h:
        s_j   = scale * q[r, h] . kv[p_j]
        o     = sum_j exp(s_j - m) kv[p_j] / sum_j exp(s_j - m),   m = max_j s_j
        lse   = m + log(sum_j exp(s_j - m))                (= log sum_j exp s_j)
    A row with no listed slot gives o = 0 and lse = -inf.
    Returns (o float64 [rows, H, D], lse float64 [rows, H]).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    slots = np.asarray(slots)
    rows, H, D = q.shape
    out = np.zeros((rows, H, D), dtype=np.float64)
    lse = np.full((rows, H), -np.inf, dtype=np.float64)
    for r in range(rows):
        sel = slots[r][slots[r] >= 0].astype(np.int64)
        if sel.size == 0:
            continue
        x = kv[sel]                                   # [n, D]
        s = float(scale) * (q[r] @ x.T)               # [H, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        out[r] = (e @ x) / z
        lse[r] = (m + np.log(z))[:, 0]
    return out, lse


def merge_attention(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint slot sets from each set's output and
    log-sum-exp: weights exp(lse_i - lse) with lse = log(exp lse1 + exp lse2)."""
    o1, o2 = np.asarray(o1, np.float64), np.asarray(o2, np.float64)
    lse1, lse2 = np.asarray(lse1, np.float64), np.asarray(lse2, np.float64)
    m = np.maximum(lse1, lse2)
    safe = np.where(np.isfinite(m), m, 0.0)
    w1, w2 = np.exp(lse1 - safe), np.exp(lse2 - safe)
    z = w1 + w2
    lse = np.where(np.isfinite(m), safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    zz = np.where(z > 0, z, 1.0)[..., None]
    return (w1[..., None] * o1 + w2[..., None] * o2) / zz, lse
