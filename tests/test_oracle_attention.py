"""Pins of the oracle's sparse attention over selected slots: torch's own
scaled-dot-product attention (float64, CPU) on the gathered rows, closed forms, the
dense case, invariances, and the log-sum-exp merge of disjoint sets."""
import math

import numpy as np
import torch

from oracle import oracle as O

D = 512


def _sdpa(q, kv, sel, scale):
    """torch.nn.functional.scaled_dot_product_attention with key = value = the
    gathered rows, float64 on the CPU: [H, D]."""
    x = torch.from_numpy(kv[sel]).unsqueeze(0)                    # [1, n, D]
    qq = torch.from_numpy(q).unsqueeze(1)                         # [H, 1, D]
    xx = x.expand(q.shape[0], -1, -1).contiguous()                # [H, n, D]
    return torch.nn.functional.scaled_dot_product_attention(qq, xx, xx, scale=scale)[:, 0].numpy()


def test_matches_torch_sdpa_on_the_gathered_rows():
    rng = np.random.default_rng(0)
    rows, H, k, n_slots = 5, 16, 37, 300
    q = rng.standard_normal((rows, H, D))
    kv = rng.standard_normal((n_slots, D))
    slots = np.full((rows, k), -1, np.int64)
    for r in range(rows):
        m = [37, 1, 20, 5, 36][r]
        slots[r, :m] = rng.choice(n_slots, m, replace=False)
        rng.shuffle(slots[r])                                     # padding anywhere in the list
    scale = 1 / math.sqrt(D)
    o, lse = O.sparse_attention(q, kv, slots, scale)
    for r in range(rows):
        sel = slots[r][slots[r] >= 0]
        want = _sdpa(q[r], kv, sel, scale)
        assert np.allclose(o[r], want, rtol=1e-12, atol=1e-13)
        s = scale * q[r] @ kv[sel].T
        assert np.allclose(lse[r], np.log(np.exp(s).sum(axis=1)), rtol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(1)
    H, n_slots = 8, 50
    q = rng.standard_normal((3, H, D))
    kv = rng.standard_normal((n_slots, D))
    scale = 0.05
    # one listed slot: the output is that row, lse its score
    o, lse = O.sparse_attention(q[:1], kv, np.array([[-1, 17, -1]]), scale)
    assert np.array_equal(o[0], np.repeat(kv[17][None], H, 0))
    assert np.allclose(lse[0], scale * q[0] @ kv[17], rtol=1e-14)
    # zero query: uniform weights, the mean of the listed rows, lse = log n
    sel = np.array([3, 9, 10, 44])
    o, lse = O.sparse_attention(np.zeros((1, H, D)), kv, sel[None], scale)
    assert np.allclose(o[0], np.repeat(kv[sel].mean(0)[None], H, 0), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse[0], math.log(4), rtol=1e-14)
    # nothing listed: zeros and -inf
    o, lse = O.sparse_attention(q[:1], kv, np.full((1, 6), -1), scale)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # a slot listed twice counts twice: same as doubling its weight
    o2, _ = O.sparse_attention(q[:1], kv, np.array([[5, 5, 8]]), scale)
    s = scale * q[0] @ kv[[5, 8]].T
    w = np.exp(s - s.max(1, keepdims=True)) * np.array([2.0, 1.0])
    assert np.allclose(o2[0], (w @ kv[[5, 8]]) / w.sum(1, keepdims=True), rtol=1e-13)


def test_every_slot_listed_is_dense_attention():
    rng = np.random.default_rng(2)
    H, n = 4, 120
    q = rng.standard_normal((1, H, D))
    kv = rng.standard_normal((n, D))
    o, _ = O.sparse_attention(q, kv, np.arange(n)[None], 0.04)
    dense = torch.softmax(torch.from_numpy(0.04 * q[0] @ kv.T), dim=-1).numpy() @ kv
    assert np.allclose(o[0], dense, rtol=1e-12, atol=1e-14)


def test_invariant_to_the_order_of_the_list():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, D))
    kv = rng.standard_normal((64, D))
    sl = np.concatenate([rng.choice(64, 20, replace=False), -np.ones(5, np.int64)])
    a = O.sparse_attention(q, kv, sl[None], 0.1)
    rng.shuffle(sl)
    b = O.sparse_attention(q, kv, sl[None], 0.1)
    assert np.allclose(a[0], b[0], rtol=1e-13) and np.allclose(a[1], b[1], rtol=1e-14)


def test_merge_of_disjoint_sets_is_attention_over_their_union():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 8, D))
    kv = rng.standard_normal((200, D)) * 2
    perm = rng.permutation(200)
    s1, s2 = perm[:70], perm[70:150]
    scale = 1 / math.sqrt(D)
    o1, l1 = O.sparse_attention(q, kv, np.stack([s1, s1]), scale)
    o2, l2 = O.sparse_attention(q, kv, np.stack([s2, s2]), scale)
    o, lse = O.sparse_attention(q, kv, np.stack([perm[:150], perm[:150]]), scale)
    om, lm = O.merge_attention(o1, l1, o2, l2)
    assert np.allclose(om, o, rtol=1e-12, atol=1e-13) and np.allclose(lm, lse, rtol=1e-13)
    # merging with an empty set changes nothing
    oe, le = O.sparse_attention(q, kv, np.full((2, 3), -1), scale)
    om2, lm2 = O.merge_attention(o, lse, oe, le)
    assert np.allclose(om2, o, rtol=1e-14) and np.array_equal(lm2, lse)


def test_a_needle_the_selection_drops_is_invisible_to_sparse_attention():
    # Dense attention (every row listed) recalls a strongly matching row; sparse
    # attention sees it only if the selection keeps it ("Root cause found": invisible
    # in dense, fatal in sparse).
    rng = np.random.default_rng(5)
    n, H = 4000, 4
    kv = rng.standard_normal((n, D))
    q = rng.standard_normal((1, H, D))
    needle = 4000 // 2
    kv[needle] = 3.0 * q[0].mean(0) / np.linalg.norm(q[0].mean(0)) * math.sqrt(D)
    scale = 1 / math.sqrt(D)
    dense, _ = O.sparse_attention(q, kv, np.arange(n)[None], scale)
    with_needle = np.concatenate([[needle], rng.choice(np.delete(np.arange(n), needle), 511, replace=False)])
    without = with_needle[1:]
    o_in, _ = O.sparse_attention(q, kv, with_needle[None], scale)
    o_out, _ = O.sparse_attention(q, kv, without[None], scale)
    u = kv[needle] / np.linalg.norm(kv[needle])
    along = lambda o: float(np.mean(o[0] @ u)) / np.linalg.norm(kv[needle])
    assert along(dense) > 0.5 and along(o_in) > 0.5      # the needle dominates the output
    assert abs(along(o_out)) < 0.1                        # gone without it
