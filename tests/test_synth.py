"""The seeded generators: determinism and the structure of each workload."""
import numpy as np

from synth import gen


def test_deterministic_and_seed_sensitive():
    a, b = gen.config(2, scale=0.05), gen.config(2, scale=0.05)
    assert np.array_equal(a.q_bits, b.q_bits) and np.array_equal(a.block_table, b.block_table)
    assert all(np.array_equal(x, y) for x, y in zip(a.keys_bits, b.keys_bits))
    c = gen.config(2, scale=0.05, seed=1)
    assert not np.array_equal(a.q_bits, c.q_bits)


def test_page_table_is_a_permutation_of_the_pool():
    wl = gen.config(2, scale=0.05)
    used = np.concatenate([wl.block_table[b, :(int(n) + wl.block_size - 1) // wl.block_size]
                           for b, n in enumerate(wl.seq_len)])
    assert np.array_equal(np.sort(used), np.arange(wl.num_blocks))
    x, slots = wl.prefix_tokens()
    assert np.unique(slots).size == slots.size
    assert np.intersect1d(slots, wl.new_slots()).size == 0


def test_workload_shapes():
    w1 = gen.config(1)
    assert w1.rows == 1 and w1.max_row_len == 2000 and w1.needle_pos[0] == 1100 and w1.k == 512
    w2 = gen.config(2, scale=0.05)
    assert w2.rows == 32 and w2.new_x_bits.shape == (32, 128) and np.all(w2.new_pos == w2.seq_len - 1)
    d = w2.needle_pos / w2.stored_len
    assert np.all((d >= 0.39) & (d <= 0.61))
    w4 = gen.config(4, scale=0.02)
    m = w4.rows
    assert np.array_equal(w4.row_len, w4.seq_len[0] - m + np.arange(m) + 1)
    w5 = gen.config(5, scale=0.001)
    assert w5.new_x_bits.shape[0] == 4 * int(w5.seq_len[0] - w5.stored_len[0])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.0], np.float32)
    got = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.0]
