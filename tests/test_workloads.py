"""Seeded input generators: determinism and the structure each workload promises."""
import numpy as np

import workloads as wl


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -2.5, 3.0e38, 0.0], np.float32)
    bits = wl.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: round to even mantissa (1.0)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80
    # 1 + 1.5 * 2^-8 rounds up to 1 + 2^-7
    assert bits[2] == 0x3F81
    assert wl.bf16_bits_to_f32(bits)[4] == -2.5
    assert np.isnan(wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_determinism_and_order():
    a = wl.config(1)
    b = wl.config(1)
    for f in ("q", "k_pool", "v_pool", "block_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = wl.config(1, seed=99)
    assert not np.array_equal(a.k_pool, c.k_pool)
    s = wl.config(4, values=False)
    assert np.array_equal(s.block_table, wl.config(4, values=False).block_table)


def test_config_shapes():
    c1 = wl.config(1, values=False)
    assert c1.num_pool_blocks == 6 and (c1.seq_len == 48).all() and (c1.q_start == 47).all()
    assert len(np.unique(c1.block_table[:, :2])) == 2        # two shared prefix blocks
    c2 = wl.config(2, values=False)
    assert c2.num_seqs == 64 and c2.seq_len.min() >= 512 and c2.seq_len.max() <= 4096
    assert (c2.q_start == c2.seq_len - 1).all() and (c2.q_len == 1).all()
    c3 = wl.config(3, values=False)
    assert c3.num_rows == 32768 and c3.num_pool_blocks == 2176
    assert (c3.block_table[:, :128] == c3.block_table[0, :128]).all()
    c4 = wl.config(4, values=False)
    assert c4.num_rows == 16 * 512 + 96 + 32 * 5
    assert (c4.q_len[:16] == 512).all() and (c4.q_len[16:112] == 1).all() and (c4.q_len[112:] == 5).all()
    c5 = wl.config(5, values=False)
    assert c5.num_pool_blocks == 10240 and c5.num_kv_splits == 16
    for p in range(4):
        a, b = c5.block_table[2 * p], c5.block_table[2 * p + 1]
        assert (a[:1536] == b[:1536]).all() and not np.intersect1d(a[1536:], b[1536:]).size


def test_tables_are_permutations_of_the_pool():
    for i in (2, 3, 4, 5):
        b = wl.config(i, values=False)
        used = set()
        for s in range(b.num_seqs):
            nb = -(-int(b.seq_len[s]) // 16)
            used.update(b.block_table[s, :nb].tolist())
            assert (b.block_table[s, nb:] == -1).all()
        assert used == set(range(b.num_pool_blocks))


def test_algorithmic_counts_config1():
    w = wl.algorithmic_work(wl.config(1, values=False))
    assert w["unique_kv_tokens"] == 32 + 4 * 16 and w["logical_kv_tokens"] == 4 * 48
    assert w["visible_pairs"] == 4 * 48 and w["flop"] == 4 * 64 * 1 * 192


def test_subset_keeps_rows_and_pool():
    """A class-only sub-batch carries its sequences' rows unchanged, so the
    oracle gives it exactly the rows the whole batch gives them."""
    import oracle
    b = wl.custom([dict(q_len=1, seq_len=40, q_start=39), dict(q_len=5, seq_len=30, q_start=25),
                   dict(q_len=20, seq_len=50, q_start=30), dict(q_len=1, seq_len=17, q_start=16)],
                  hq=4, hkv=2, d=8, dtype="bf16", seed=3)
    kinds = [wl.seq_kind(int(n)) for n in b.q_len]
    assert kinds == ["decode", "verify", "prefill", "decode"]
    full_o, full_l = oracle.attend(b)
    off = b.row_offsets()
    for kind in ("decode", "verify", "prefill"):
        keep = np.array([k == kind for k in kinds])
        sb = wl.subset(b, keep, kind)
        assert sb.k_pool is b.k_pool and sb.num_pool_blocks == b.num_pool_blocks
        rows = np.concatenate([np.arange(off[s], off[s + 1]) for s in np.nonzero(keep)[0]])
        o, lse = oracle.attend(sb)
        np.testing.assert_array_equal(o, full_o[rows])
        np.testing.assert_array_equal(lse, full_l[rows])
