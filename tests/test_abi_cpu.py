"""The C ABI on a machine without a GPU: the library loads, exports every entry point
include/dsa_indexer.h declares, and rejects bad arguments on the host before any
launch (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import sparse_attention_token_store_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = dsa.load_library()
    names = declared_functions()
    assert set(names) == set(dsa.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.indexer_abi_version() == 2


FAKE = 1 << 20          # never dereferenced: every call below fails validation first
ALIGNED = 1 << 24


def cache(dtype=dsa.IDX_FP8_E4M3, bs=64, nb=10, base=ALIGNED):
    return dsa.KCache(base, dtype, bs, nb)


def rows(n=4, max_row_len=100, max_blocks=4, num_seqs=2):
    return dsa.Rows(FAKE, max_blocks, num_seqs, FAKE, FAKE, n, max_row_len)


def err(lib):
    return lib.indexer_last_error().decode()


def test_store_validation():
    lib = dsa.load_library()
    f = lib.index_k_store
    assert f(FAKE, -1, None, FAKE, cache(), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert f(FAKE, 4, None, FAKE, cache(), 8, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert "flag" in err(lib)
    assert f(FAKE, 4, None, FAKE, cache(base=ALIGNED + 16), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert "aligned" in err(lib)
    assert f(FAKE, 4, None, FAKE, cache(bs=16), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_EUNSUPPORTED
    assert f(FAKE, 4, None, FAKE, cache(dtype=4), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert f(FAKE, 4, FAKE, FAKE, cache(), dsa.IDX_STORE_ROPE, 1e-6, 1e4, 63, None, None) == dsa.IDX_EINVAL
    assert "rope_dim" in err(lib)
    assert f(FAKE, 4, FAKE, FAKE, cache(), dsa.IDX_STORE_ROPE, 1e-6, -1.0, 64, None, None) == dsa.IDX_EINVAL
    assert f(FAKE, 4, None, FAKE, cache(), dsa.IDX_STORE_ROPE, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert "positions" in err(lib)
    assert f(FAKE, 4, None, FAKE, cache(), dsa.IDX_STORE_RMSNORM, -1.0, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert f(None, 4, None, FAKE, cache(), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert f(FAKE + 2, 4, None, FAKE, cache(), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    assert f(FAKE, 4, None, FAKE + 4, cache(), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_EINVAL
    # n = 0 is a no-op that never touches the GPU
    assert f(None, 0, None, None, cache(), 0, 1e-6, 1e4, 64, None, None) == dsa.IDX_OK
    assert err(lib) == ""


def test_q_prep_validation():
    lib = dsa.load_library()
    f = lib.indexer_q_prep
    R, H = dsa.IDX_STORE_ROPE, dsa.IDX_STORE_HADAMARD
    ok = (FAKE, 8, 4, FAKE, R | H, 1e-6, 1e4, 64, FAKE, None, None, None, None)
    def call(**kw):
        names = ("q", "n", "heads", "pos", "flags", "eps", "base", "rope_dim", "out", "codes", "scales", "dbg", "s")
        a = dict(zip(names, ok))
        a.update(kw)
        return f(*[a[n] for n in names])
    assert call(n=-1) == dsa.IDX_EINVAL
    assert call(heads=0) == dsa.IDX_EINVAL
    assert call(n=7) == dsa.IDX_EINVAL and "multiple" in err(lib)
    assert call(flags=8) == dsa.IDX_EINVAL and "flag" in err(lib)
    assert call(rope_dim=63) == dsa.IDX_EINVAL and "rope_dim" in err(lib)
    assert call(base=0.0) == dsa.IDX_EINVAL
    assert call(flags=dsa.IDX_STORE_RMSNORM, eps=-1.0) == dsa.IDX_EINVAL
    assert call(codes=FAKE) == dsa.IDX_EINVAL and "together" in err(lib)
    assert call(out=None) == dsa.IDX_EINVAL and "output" in err(lib)
    assert call(q=None) == dsa.IDX_EINVAL
    assert call(q=FAKE + 2) == dsa.IDX_EINVAL and "aligned" in err(lib)
    assert call(pos=None) == dsa.IDX_EINVAL and "positions" in err(lib)
    assert call(out=FAKE + 2) == dsa.IDX_EINVAL
    assert call(out=None, codes=FAKE + 1, scales=FAKE) == dsa.IDX_EINVAL
    assert call(out=None, codes=FAKE, scales=FAKE + 2) == dsa.IDX_EINVAL
    assert call(dbg=FAKE + 4) == dsa.IDX_EINVAL
    # the kernel moves 16-byte chunks of q, out_bf16 and prequant_dbg and 8-byte
    # chunks of codes: those alignments are required
    assert call(q=FAKE + 8) == dsa.IDX_EINVAL and "q_bf16" in err(lib)
    assert call(out=FAKE + 8) == dsa.IDX_EINVAL and "out_bf16" in err(lib)
    assert call(out=None, codes=FAKE + 4, scales=FAKE) == dsa.IDX_EINVAL and "codes" in err(lib)
    assert call(dbg=FAKE + 8) == dsa.IDX_EINVAL and "prequant_dbg" in err(lib)
    # no RoPE: positions may be NULL; n = 0 is a no-op that never touches the GPU
    assert call(n=0, q=None, pos=None, flags=H) == dsa.IDX_OK
    assert call(n=0, q=None, pos=None, out=None, flags=H) == dsa.IDX_OK   # (empty outputs: NULL)
    assert err(lib) == ""


def test_quant_validation():
    lib = dsa.load_library()
    f = lib.indexer_quant_fp8
    assert f(FAKE, -3, FAKE, FAKE, None) == dsa.IDX_EINVAL
    assert f(None, 3, FAKE, FAKE, None) == dsa.IDX_EINVAL
    assert f(FAKE + 8, 3, FAKE, FAKE, None) == dsa.IDX_EINVAL
    assert f(FAKE, 3, FAKE + 4, FAKE, None) == dsa.IDX_EINVAL
    assert f(FAKE, 0, None, None, None) == dsa.IDX_OK


def test_score_validation():
    lib = dsa.load_library()
    f = lib.indexer_score
    ok = dict(q=FAKE, qd=dsa.IDX_BF16, qs=None, w=FAKE, h=64, c=cache(), r=rows(), s=FAKE, ld=128)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["q"], a["qd"], a["qs"], a["w"], a["h"], a["c"], a["r"], a["s"], a["ld"], None)

    assert call(h=32) == dsa.IDX_EUNSUPPORTED and "heads" in err(lib)
    assert call(qd=dsa.IDX_FP8_E4M3, c=cache(dtype=dsa.IDX_BF16), qs=FAKE) == dsa.IDX_EUNSUPPORTED
    assert call(c=cache(dtype=4)) == dsa.IDX_EINVAL
    assert call(qd=dsa.IDX_FP8_E4M3) == dsa.IDX_EINVAL and "q_scale" in err(lib)
    assert call(qd=7) == dsa.IDX_EINVAL
    assert call(ld=99) == dsa.IDX_EINVAL and "ld" in err(lib)
    assert call(r=rows(max_row_len=300)) == dsa.IDX_EINVAL          # > max_blocks * block_size
    assert call(r=rows(n=70000)) == dsa.IDX_EINVAL
    assert call(r=rows(n=-1)) == dsa.IDX_EINVAL
    assert call(q=FAKE + 8) == dsa.IDX_EINVAL
    assert call(s=None) == dsa.IDX_EINVAL
    assert call(c=cache(nb=0)) == dsa.IDX_EINVAL
    assert call(r=dsa.Rows(None, 4, 2, FAKE, FAKE, 4, 100)) == dsa.IDX_EINVAL
    assert call(r=rows(n=0)) == dsa.IDX_OK


def test_topk_validation_and_workspace():
    lib = dsa.load_library()
    f = lib.indexer_topk
    assert f(FAKE, 100, FAKE, 4, 100, 0, FAKE, None, 0, None) == dsa.IDX_EINVAL
    assert f(FAKE, 100, FAKE, 4, 100, 8193, FAKE, None, 0, None) == dsa.IDX_EINVAL
    assert f(FAKE, 99, FAKE, 4, 100, 8, FAKE, None, 0, None) == dsa.IDX_EINVAL
    assert f(FAKE, 100, None, 4, 100, 8, FAKE, None, 0, None) == dsa.IDX_EINVAL
    # long rows need a workspace; too small is refused before any launch
    need = lib.indexer_workspace_bytes(dsa.IDX_OP_TOPK, 4, 1 << 20, 1024)
    assert need > 0
    assert lib.indexer_workspace_bytes(dsa.IDX_OP_TOPK, 4, 20000, 512) == 0
    assert f(FAKE, 1 << 20, FAKE, 4, 1 << 20, 1024, FAKE, ALIGNED, need - 1, None) == dsa.IDX_EWORKSPACE
    assert f(FAKE, 1 << 20, FAKE, 4, 1 << 20, 1024, FAKE, ALIGNED + 64, need, None) == dsa.IDX_EINVAL
    st = lib.indexer_score_topk
    need2 = lib.indexer_workspace_bytes(dsa.IDX_OP_SCORE_TOPK, 4, 100, 8)
    assert need2 >= 4 * 128 * 4
    assert st(FAKE, dsa.IDX_BF16, None, FAKE, 64, cache(), rows(), 8, FAKE, None, None, ALIGNED, need2 - 1, None) == dsa.IDX_EWORKSPACE
    assert st(FAKE, dsa.IDX_BF16, None, FAKE, 64, cache(), rows(), 0, FAKE, None, None, ALIGNED, need2, None) == dsa.IDX_EINVAL
    # out_slots must be 8-byte aligned
    assert st(FAKE, dsa.IDX_BF16, None, FAKE, 64, cache(), rows(), 8, FAKE, FAKE + 4, None, ALIGNED, need2, None) == dsa.IDX_EINVAL
    assert "out_slots" in err(lib)
    assert lib.indexer_workspace_bytes(99, 4, 100, 8) == 0
    assert lib.indexer_workspace_bytes(dsa.IDX_OP_TOPK, 4, 100, 0) == 0


def test_topk_plan_at_the_largest_sizes():
    # the longest rows the ABI accepts need the most reduction levels (k = 8192 keeps
    # half of each first-level chunk); the host-side plan must size them without
    # overrunning its tables, and the workspace must cover two candidate lists of
    # the first level's survivors
    # The plan: first-level chunks of 16,384 (doubled until >= 2k), or twice that where
    # it saves a whole level; later levels of 8k (a power of two, at most 32,768) until
    # one 36,864-element chunk is left.
    def after(m, c, k):
        return (m // c) * min(k, c) + min(m % c, k)

    def levels(n, k, first):
        c0 = first
        while c0 < 2 * k:
            c0 *= 2
        m, lv, c = n, 0, c0
        while m > 36864:
            m = after(m, c, k)
            lv += 1
            c = 4096
            while c < 8 * k and c < 32768:
                c *= 2
        return lv + 1, c0

    lib = dsa.load_library()
    for rows, n, k in [(1, 2**31 - 1, 8192), (1, 2**31 - 1, 1), (3, 2**31 - 1, 4097),
                       (65535, 2**31 - 1, 8192), (1, 36865, 8192), (1, 1 << 20, 8192),
                       (4, 1 << 20, 1024), (16, 131072, 1024)]:
        need = lib.indexer_workspace_bytes(dsa.IDX_OP_TOPK, rows, n, k)
        la, ca = levels(n, k, 16384)
        lb, cb = levels(n, k, 32768)
        chunk0 = cb if la > 2 and lb < la else ca
        survivors = after(n, chunk0, k)
        assert need >= 2 * rows * survivors * 8, (rows, n, k, need)
        assert need == lib.indexer_workspace_bytes(dsa.IDX_OP_TOPK, rows, n, k)   # deterministic
        both = lib.indexer_workspace_bytes(dsa.IDX_OP_SCORE_TOPK, rows, n, k)
        assert both == 0 or both > need


def test_error_string_is_thread_local():
    import threading
    lib = dsa.load_library()
    out = {}

    def worker():
        lib.indexer_quant_fp8(FAKE, -1, FAKE, FAKE, None)
        out["t"] = err(lib)

    lib.indexer_quant_fp8(FAKE, 0, None, None, None)   # success clears this thread's error
    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert "n_vec" in out["t"]
    assert err(lib) == ""


def test_translate_validation():
    lib = dsa.load_library()
    f = lib.indexer_translate
    ok = dict(idx=FAKE, ld_idx=8, k=8, cache=cache(), rows=rows(), slots=FAKE, ld_slots=8)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["idx"], a["ld_idx"], a["k"], a["cache"], a["rows"], a["slots"], a["ld_slots"], None)

    assert call(k=-1) == dsa.IDX_EINVAL
    assert call(ld_idx=7) == dsa.IDX_EINVAL
    assert call(ld_slots=7) == dsa.IDX_EINVAL
    assert call(cache=cache(bs=16)) == dsa.IDX_EUNSUPPORTED
    assert call(cache=cache(nb=0)) == dsa.IDX_EINVAL
    assert call(idx=None) == dsa.IDX_EINVAL
    assert call(slots=None) == dsa.IDX_EINVAL
    assert call(idx=FAKE + 2) == dsa.IDX_EINVAL and "idx" in err(lib)
    assert call(slots=FAKE + 4) == dsa.IDX_EINVAL and "slots" in err(lib)
    # the cache base is not read: NULL is accepted by validation (checked here with a
    # misaligned slots pointer, so nothing is launched)
    assert call(cache=cache(base=None), slots=FAKE + 4) == dsa.IDX_EINVAL and "slots" in err(lib)
    # nothing to do: no launch, no pointer needed
    assert call(k=0, idx=None, slots=None) == dsa.IDX_OK
    assert call(rows=rows(n=0), idx=None, slots=None) == dsa.IDX_OK


def test_sparse_attention_validation_and_workspace():
    lib = dsa.load_library()
    f = lib.indexer_sparse_attention
    ws_of = lib.indexer_attention_workspace_bytes
    need = ws_of(32, 512, 16)
    assert need > 0 and ws_of(32, 512, 16) == dsa.attention_workspace_bytes(32, 512, 16)
    # (the partial outputs and (max, log-sum) pairs of every split are fp32)
    assert need % (32 * 16 * (dsa.KV_DIM + 2) * 4) == 0
    for bad in [(-1, 512, 16), (65536, 512, 16), (32, -1, 16), (32, (1 << 16) + 1, 16), (32, 512, 24)]:
        assert ws_of(*bad) == 0, bad
    assert ws_of(0, 512, 16) == 0

    ok = dict(q=FAKE, heads=16, kv=ALIGNED, num_slots=1000, slots=FAKE, ld_slots=512, k=512, rows=32,
              scale=0.04, out=ALIGNED, lse=None, ws=None, ws_bytes=0)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["q"], a["heads"], a["kv"], a["num_slots"], a["slots"], a["ld_slots"], a["k"], a["rows"],
                 a["scale"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)

    # every call below fails validation, so nothing is launched
    assert call(heads=24) == dsa.IDX_EUNSUPPORTED and "heads" in err(lib)
    assert call(rows=-1) == dsa.IDX_EINVAL
    assert call(rows=65536) == dsa.IDX_EINVAL
    assert call(k=-1) == dsa.IDX_EINVAL
    assert call(k=(1 << 16) + 1, ld_slots=1 << 17) == dsa.IDX_EINVAL
    assert call(ld_slots=511) == dsa.IDX_EINVAL and "ld_slots" in err(lib)
    assert call(num_slots=0) == dsa.IDX_EINVAL
    assert call(num_slots=1 << 31) == dsa.IDX_EINVAL
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert call(scale=s) == dsa.IDX_EINVAL and "scale" in err(lib)
    assert call(q=None) == dsa.IDX_EINVAL
    assert call(kv=None) == dsa.IDX_EINVAL
    assert call(out=None) == dsa.IDX_EINVAL
    assert call(slots=None) == dsa.IDX_EINVAL
    assert call(q=FAKE + 8) == dsa.IDX_EINVAL and "aligned" in err(lib)
    assert call(kv=ALIGNED + 4) == dsa.IDX_EINVAL
    assert call(out=ALIGNED + 8) == dsa.IDX_EINVAL
    assert call(slots=FAKE + 4) == dsa.IDX_EINVAL and "slots" in err(lib)
    assert call(lse=FAKE + 2) == dsa.IDX_EINVAL and "lse" in err(lib)
    # a call that needs partials: no workspace, a short one, a misaligned one
    assert call() == dsa.IDX_EWORKSPACE
    assert call(ws=ALIGNED, ws_bytes=need - 1) == dsa.IDX_EWORKSPACE
    assert call(ws=ALIGNED + 64, ws_bytes=need) == dsa.IDX_EINVAL and "256" in err(lib)
    # nothing to do: no launch, no pointer needed
    assert call(rows=0, q=None, kv=None, slots=None, out=None) == dsa.IDX_OK


def test_static_scratch_entry_point_validation():
    # the allocation-free variant runs the same argument checks as indexer_score_topk
    # and refuses, before touching the GPU, any call whose workspace would not fit the
    # static scratch array
    lib = dsa.load_library()
    f = lib.indexer_score_topk_static
    assert f(FAKE, dsa.IDX_BF16, None, FAKE, 64, cache(), rows(), 0, FAKE, None, None, None) == dsa.IDX_EINVAL
    assert f(FAKE, dsa.IDX_BF16, None, FAKE, 32, cache(), rows(), 8, FAKE, None, None, None) == dsa.IDX_EUNSUPPORTED
    assert f(FAKE, dsa.IDX_BF16, None, FAKE, 64, cache(), rows(), 8, FAKE, FAKE + 4, None, None) == dsa.IDX_EINVAL
    assert f(FAKE, dsa.IDX_BF16, None, FAKE, 64, cache(), rows(n=0), 8, FAKE, None, None, None) == dsa.IDX_OK
    # 16 rows of 1M keys need ~70 MB of scores: more than the 32 MiB the array holds
    big = dsa.Rows(FAKE, 1 << 14, 16, FAKE, FAKE, 16, 1 << 20)
    need = lib.indexer_workspace_bytes(dsa.IDX_OP_SCORE_TOPK, 16, 1 << 20, 1024)
    assert need > dsa.IDX_STATIC_SCRATCH_BYTES
    assert f(FAKE, dsa.IDX_BF16, None, FAKE, 64, cache(nb=1 << 18), big, 1024, FAKE, None, None, None) == \
        dsa.IDX_EWORKSPACE
    assert "static scratch" in err(lib) and str(dsa.IDX_STATIC_SCRATCH_BYTES) in err(lib)
    # the long-decode and decode-batch shapes fit
    assert lib.indexer_workspace_bytes(dsa.IDX_OP_SCORE_TOPK, 4, 1 << 20, 1024) <= dsa.IDX_STATIC_SCRATCH_BYTES
    assert lib.indexer_workspace_bytes(dsa.IDX_OP_SCORE_TOPK, 32, 22000, 512) <= dsa.IDX_STATIC_SCRATCH_BYTES
    header = open(HEADER).read()
    assert re.search(r"#define IDX_STATIC_SCRATCH_BYTES \(32u << 20\)", header)
