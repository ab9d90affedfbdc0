"""The fp64 oracle against closed forms, library routines, mpmath and invariants."""
import numpy as np
import pytest

import oracle
import oracle_pins as P
import workloads as wl


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.attend)


def test_split_merge_equals_unsplit():
    """Online softmax / split-KV equals softmax (XY-Serve review, "Assumptions &
    free parameters"); merge of all-empty partitions is 0 / -inf."""
    P.pin_split_merge(oracle)
    o1, l1 = oracle.merge_partitions(np.ones((1, 2, 4)), np.zeros((1, 2)))
    assert np.all(o1 == 1) and np.all(l1 == 0)
    oe, le = oracle.merge_partitions(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def test_empty_partition_is_neutral():
    b = wl.custom([dict(q_len=2, seq_len=40, q_start=38)], hq=2, hkv=1, d=8, seed=2)
    o, l = oracle.attend_partitioned(b, [45], [60])   # beyond every row: empty
    assert np.all(o == 0) and np.all(np.isneginf(l))
    o, l = oracle.attend_partitioned(b, [39], [40])   # only the second row sees key 39
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0])) and np.all(np.isfinite(l[1]))


def test_partition_bounds_reading():
    pb = oracle.partition_bounds(100, 3)          # 7 blocks -> chunk 3 blocks = 48 keys
    assert pb.tolist() == [[0, 48], [48, 96], [96, 100]]
    pb = oracle.partition_bounds(32768, 16)
    assert (pb[:, 1] - pb[:, 0] == 2048).all() and pb[-1, 1] == 32768
    pb = oracle.partition_bounds(20, 4)           # 2 blocks, chunk 1 -> two empty tails
    assert pb.tolist() == [[0, 16], [16, 20], [20, 20], [20, 20]]
    for n in range(1, 200, 7):
        for p in (1, 2, 5, 16):
            pb = oracle.partition_bounds(n, p)
            assert pb[0, 0] == 0 and pb[-1, 1] == n
            nonempty = pb[:, 0] < pb[:, 1]
            assert (pb[1:, 0] == pb[:-1, 1]).all() and (pb[nonempty, 0] % 16 == 0).all()


def test_poison_outside_visible_slots_is_ignored():
    """Slots no row may see can hold NaN or huge values without changing anything
    (XY-Serve review, "Assumptions & free parameters": padded entries do not
    affect the output)."""
    b = wl.custom([dict(q_len=3, seq_len=37, q_start=30), dict(q_len=1, seq_len=21, q_start=9)],
                  hq=4, hkv=2, d=16, seed=8, extra_blocks=2)
    ref_o, ref_l = oracle.attend(b)
    for val in (float("nan"), 6e4, -6e4):
        o, l = oracle.attend(wl.with_poison(b, val))
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)
    assert wl.visible_slot_mask(b).sum() < b.num_pool_blocks * 16


def test_rows_subset_matches_full():
    b = wl.custom([dict(q_len=7, seq_len=50), dict(q_len=1, seq_len=9), dict(q_len=4, seq_len=64)],
                  hq=4, hkv=2, d=8, seed=4)
    o, l = oracle.attend(b)
    rows = [11, 0, 6, 8]
    o2, l2 = oracle.attend(b, rows=rows)
    assert np.allclose(o2, o[rows], rtol=0, atol=1e-15) and np.allclose(l2, l[rows], rtol=0, atol=1e-15)


def test_kv_append_pins():
    P.pin_append(oracle.append_kv, oracle.gather_kv)
