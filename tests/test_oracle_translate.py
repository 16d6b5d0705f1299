"""Pins of the oracle's logical -> physical translation (oracle.translate):
a hand-worked example with every -1 case, the closed form of an identity block
table, the slot the store was given for every stored position of a generated
workload, and injectivity over a shuffled block table."""
import numpy as np

from oracle import oracle as O
from synth import gen


def test_hand_worked_example():
    # block size 4; sequence 0 -> physical blocks (2, 0), sequence 1 -> (1, 3)
    table = np.array([[2, 0], [1, 3]])
    row_seq = np.array([1, 0])
    row_len = np.array([7, 5])
    idx = np.array([[0, 3, 4, 6, 7, -1],
                    [4, 5, 0, -1, 2, 100]])
    # row 0 (sequence 1, 7 keys): 0 -> block 1 -> 4; 3 -> 7; 4 -> block 3 -> 12;
    # 6 -> 14; 7 is not visible; -1 is padding
    # row 1 (sequence 0, 5 keys): 4 -> block 0 -> 0; 5 not visible; 0 -> block 2 -> 8;
    # 2 -> 10; 100 past the row
    want = np.array([[4, 7, 12, 14, -1, -1],
                     [0, -1, 8, -1, 10, -1]])
    assert np.array_equal(O.translate(idx, table, row_seq, row_len, 4, 4), want)
    # max_row_len cuts the visible range; a block id outside the pool and a sequence
    # id outside the table give -1
    assert np.array_equal(O.translate(idx, table, row_seq, row_len, 4, 4, max_row_len=4)[0],
                          [4, 7, -1, -1, -1, -1])
    bad = np.array([[2, 9], [1, -3]])
    assert np.array_equal(O.translate(idx, bad, row_seq, row_len, 4, 4),
                          [[4, 7, -1, -1, -1, -1], [-1, -1, 8, -1, 10, -1]])
    assert np.all(O.translate(idx, table, np.array([2, -1]), row_len, 4, 4) == -1)
    # a logical block past the table's width
    assert O.translate(np.array([[8]]), table, [0], [100], 4, 4)[0, 0] == -1


def test_identity_table_closed_form():
    # block_table[s][j] = s * max_blocks + j makes the slot s * max_blocks * bs + t
    rng = np.random.default_rng(0)
    num_seqs, max_blocks = 5, 7
    for bs in (32, 64):
        table = np.arange(num_seqs * max_blocks).reshape(num_seqs, max_blocks)
        row_seq = rng.integers(0, num_seqs, 40)
        row_len = rng.integers(0, max_blocks * bs + 1, 40)
        idx = rng.integers(-1, max_blocks * bs, (40, 33))
        got = O.translate(idx, table, row_seq, row_len, bs, num_seqs * max_blocks)
        vis = (idx >= 0) & (idx < row_len[:, None])
        want = np.where(vis, row_seq[:, None] * max_blocks * bs + idx, -1)
        assert np.array_equal(got, want)


def test_store_slot_of_every_stored_position():
    # the generator hands the store a slot for every key it writes; the translation
    # of that key's position in its row must be that slot
    wl = gen.config(2, scale=0.01)
    _, slots = wl.prefix_tokens()
    off = 0
    for b, kb in enumerate(wl.keys_bits):
        n = kb.shape[0]
        got = O.translate(np.arange(n)[None], wl.block_table, [b], [n], wl.block_size, wl.num_blocks)[0]
        assert np.array_equal(got, slots[off:off + n])
        off += n
    new = wl.new_slots()
    for i in range(new.size):
        s, p = int(wl.new_seq[i]), int(wl.new_pos[i])
        assert O.translate([[p]], wl.block_table, [s], [p + 1], wl.block_size, wl.num_blocks)[0, 0] == new[i]


def test_injective_on_a_shuffled_table():
    # distinct (sequence, position) pairs land on distinct slots of the pool
    rng = np.random.default_rng(3)
    num_seqs, max_blocks, bs = 6, 9, 32
    perm = rng.permutation(num_seqs * max_blocks + 11)[:num_seqs * max_blocks]
    table = perm.reshape(num_seqs, max_blocks)
    n = max_blocks * bs
    got = O.translate(np.tile(np.arange(n), (num_seqs, 1)), table, np.arange(num_seqs),
                      np.full(num_seqs, n), bs, num_seqs * max_blocks + 11)
    assert np.all(got >= 0) and np.unique(got).size == got.size
    assert got.max() < (num_seqs * max_blocks + 11) * bs
