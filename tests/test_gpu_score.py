"""HIP indexer_score against the oracle (C1), page-table invariance, determinism."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import GpuWorkload, i32, note
from _parity import RTOL, OracleKeys, check_scores, oracle_scores

pytestmark = pytest.mark.gpu


def gpu_scores(g: GpuWorkload, ld=None, fp8_q=False):
    wl = g.wl
    ld = ld or wl.max_row_len + 7
    out = torch.full((wl.rows, ld), 12345.0, dtype=torch.float32, device="cuda")
    q, qs = g.query(fp8_q)
    note(f"indexer_score {wl.name} {g.key_dtype} rows={wl.rows} max_len={wl.max_row_len} bs={wl.block_size}")
    dsa.indexer_score(q, g.w, g.cache, g.rows, out, q_scale=qs)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, wl.max_row_len:] == 12345.0), "columns beyond max_row_len must not be written"
    return o


CASES = [
    # config, scale, key dtype, block size
    (1, 1.0, "bf16", 64),
    (1, 1.0, "fp8", 32),
    (2, 0.1, "fp8", 64),
    (2, 0.1, "bf16", 32),
    (3, 0.02, "bf16", 64),
    (3, 0.02, "fp8", 64),
    (5, 0.004, "fp8", 64),
]


@pytest.mark.parametrize("cfg,scale,kd,bs", CASES)
def test_score_matches_oracle(cfg, scale, kd, bs):
    wl = gen.config(cfg, scale=scale, block_size=bs, key_dtype=kd if cfg != 4 else None)
    g = GpuWorkload(wl, key_dtype=kd)
    g.store_new()
    got = gpu_scores(g)
    ok = OracleKeys(wl, kd)
    o = oracle_scores(wl, ok)
    stats = check_scores(got, o, wl.row_len, RTOL[kd], slack=ok.slack())
    print(stats)


@pytest.mark.parametrize("kd", ["fp8", "bf16", "fp4"])
def test_page_table_permutation_is_bit_invariant(kd):
    # identical logical keys behind the identity table and behind a shuffled one
    wl_id = gen.config(2, scale=0.05, shuffle=False)
    wl_sh = gen.config(2, scale=0.05, shuffle=True)
    assert not np.array_equal(wl_id.block_table, wl_sh.block_table)
    a = gpu_scores(GpuWorkload(wl_id, key_dtype=kd))
    b = gpu_scores(GpuWorkload(wl_sh, key_dtype=kd))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_deterministic_and_ld_independent():
    wl = gen.config(2, scale=0.05)
    g = GpuWorkload(wl)
    a = gpu_scores(g)
    b = gpu_scores(g, ld=wl.max_row_len + 300)
    assert np.array_equal(a[:, :wl.max_row_len].view(np.uint32), b[:, :wl.max_row_len].view(np.uint32))


@pytest.mark.parametrize("kd,bs", [("fp8", 64), ("bf16", 64), ("fp4", 64), ("fp8", 32), ("bf16", 32), ("fp4", 32)])
def test_ragged_rows_and_edge_lengths(kd, bs):
    # rows of length 0, 1, 15, 16, 17, 63, 64, 65 and one spanning many blocks: a
    # workgroup's waves then hold from zero to many key groups
    lens = np.array([0, 1, 15, 16, 17, 63, 64, 65, 777], np.int64)
    wl = gen.make(np.maximum(lens, 1), key_dtype=kd, k=4, needle_depth=None, block_size=bs, seed=5)
    wl.row_len = lens.astype(np.int32)
    g = GpuWorkload(wl, key_dtype=kd)
    got = gpu_scores(g)
    o = oracle_scores(wl, OracleKeys(wl, kd))
    check_scores(got, o, wl.row_len, RTOL[kd])


def test_rows_sharing_a_sequence():
    # several query rows reading one sequence with different causal lengths
    wl = gen.make([3000], key_dtype="bf16", k=64, needle_depth=None, prefill_rows=40, seed=6)
    g = GpuWorkload(wl, key_dtype="bf16")
    got = gpu_scores(g)
    check_scores(got, oracle_scores(wl, OracleKeys(wl, "bf16")), wl.row_len, RTOL["bf16"])


@pytest.mark.parametrize("bs", [64, 32])
@pytest.mark.parametrize("case", ["bf16_keys", "fp8_keys", "fp8_prefill", "fp4_keys"])
def test_bad_block_id_scores_nan_without_faulting(case, bs):
    # a block id outside the pool is caught by the kernel's bounds check: exactly the
    # keys it covers score NaN in every row that sees them (at block size 32 the
    # other half of the 64-key span stays finite), nothing is read out of bounds
    # (one case per scoring kernel: bf16 keys, fp8 keys, fp8 queries, fp4 keys)
    wl = {"bf16_keys": lambda: gen.config(1, scale=0.2, block_size=bs),
          "fp8_keys": lambda: gen.config(2, scale=0.05, block_size=bs),
          "fp8_prefill": lambda: gen.config(4, scale=0.02, block_size=bs),
          "fp4_keys": lambda: gen.config(3, scale=0.01, block_size=bs)}[case]()
    seq = int(wl.row_seq[0])
    bt = wl.block_table.copy()
    bt[seq, 1] = wl.num_blocks + 5
    g = GpuWorkload(wl, block_table=bt, key_dtype="fp4" if case == "fp4_keys" else None)
    g.store_new()   # (decode b32 keeps each sequence's newest key for the store chain)
    if case == "fp8_prefill":
        g.quantise_q()
        got = gpu_scores(g, fp8_q=True)
    else:
        got = gpu_scores(g)
    bs = wl.block_size
    checked = 0
    for r in range(wl.rows):
        n = int(wl.row_len[r])
        if int(wl.row_seq[r]) != seq or n <= bs:
            continue
        assert np.all(np.isnan(got[r, bs:min(2 * bs, n)]))
        assert np.all(np.isfinite(got[r, :bs]))
        assert np.all(np.isfinite(got[r, 2 * bs:n]))
        checked += 1
    assert checked > 0


def test_needle_ranks_first_on_gpu_scores():
    for S in (2000, 4500, 10000, 22000):
        for kd in ("bf16", "fp8"):
            wl = gen.make([S], key_dtype=kd, k=512, seed=0, shuffle=True)
            got = gpu_scores(GpuWorkload(wl, key_dtype=kd))
            p = int(wl.needle_pos[0])
            assert O.rank_of(got[0].astype(np.float64), S, p) == 1


def oracle_fp8_q(wl):
    """The oracle's own fp8 queries: the O4 quantiser applied to the same bf16 q."""
    c, sc = O.quant_fp8(O.bf16_bits_to_f32(wl.q_bits))
    return O.dequant_fp8(c, sc)


PREFILL_CASES = [
    # scale of the chunked-prefill workload, block size
    (0.02, 64),
    (0.05, 32),
    (0.1, 64),
]


@pytest.mark.parametrize("scale,bs", PREFILL_CASES)
def test_prefill_fp8_scores_match_oracle(scale, bs):
    wl = gen.config(4, scale=scale, block_size=bs)
    g = GpuWorkload(wl)
    g.quantise_q()
    got = gpu_scores(g, fp8_q=True)
    o = oracle_scores(wl, OracleKeys(wl), q64=oracle_fp8_q(wl))
    print(check_scores(got, o, wl.row_len, RTOL["fp8"]))


def test_prefill_kernel_rows_of_different_sequences():
    # fp8 queries on the decode layout: every row reads its own sequence, so each
    # wave of the prefill kernel makes one pass per row
    wl = gen.config(2, scale=0.05)
    g = GpuWorkload(wl)
    g.store_new()
    g.quantise_q()
    got = gpu_scores(g, fp8_q=True)
    ok = OracleKeys(wl)
    o = oracle_scores(wl, ok, q64=oracle_fp8_q(wl))
    check_scores(got, o, wl.row_len, RTOL["fp8"], slack=ok.slack())


def test_prefill_ragged_row_count():
    # a row count that leaves the last workgroup with partial waves
    wl = gen.make([900], key_dtype="fp8", k=64, needle_depth=None, prefill_rows=13, seed=7)
    g = GpuWorkload(wl)
    g.quantise_q()
    got = gpu_scores(g, fp8_q=True)
    check_scores(got, oracle_scores(wl, OracleKeys(wl), q64=oracle_fp8_q(wl)), wl.row_len, RTOL["fp8"])


@pytest.mark.parametrize("kd", ["fp8", "fp4"])
def test_prefill_bad_blocks_in_whole_and_partial_stages(kd):
    # 64-token blocks: whole 256-key stages of fp8 keys take their block ids by scalar
    # loads, the last partial stage (and MXFP4 keys) per lane; a negative id in a whole stage and an id past
    # the pool in the partial stage each turn exactly their block's keys to NaN
    wl = gen.config(4, scale=0.02, block_size=64)
    seq = int(wl.row_seq[0])
    n_max = int(wl.row_len.max())
    last = (n_max - 1) // 64
    # keys are split into 8 chunks of whole 64-key spans, each scored in 256-key
    # stages; a stage is whole when it ends within the workgroup's longest row
    ck = -(-(-(-n_max // 64)) // 8) * 64

    def stage_end(p):
        c = p // ck
        return c * ck + (p - c * ck) // 256 * 256 + 256

    for n_wg in (int(wl.row_len.min()), n_max):   # every workgroup's longest row lies in this range
        assert stage_end(128) <= n_wg and stage_end(last * 64) > n_wg
    bt = wl.block_table.copy()
    bt[seq, 2] = -1
    bt[seq, last] = wl.num_blocks + 7
    g = GpuWorkload(wl, block_table=bt, key_dtype=kd)
    g.quantise_q()
    got = gpu_scores(g, fp8_q=True)
    bad = np.zeros(n_max, bool)
    bad[128:192] = True
    bad[last * 64:] = True
    checked = 0
    for r in range(wl.rows):
        n = int(wl.row_len[r])
        assert np.all(np.isnan(got[r, :n][bad[:n]])), r
        assert np.all(np.isfinite(got[r, :n][~bad[:n]])), r
        checked += int(n > last * 64)
    assert checked > 0
