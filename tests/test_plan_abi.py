"""Host planner through the C ABI (no GPU needed): tables bit-exact against the
oracle's replica, exact coverage of every visible (row, head, key), error paths,
and the exported symbol set."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle.plan_replica as R
import prefix_shared_paged_pmattn_amd as pm
import workloads as wl
from prefix_shared_paged_pmattn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def make_plan(b, **kw):
    """A plan of ``b``; the cascade is off unless asked for (cascade plans are
    checked against the replica by ``_check_cascade_plan``)."""
    return pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, num_pool_blocks=b.num_pool_blocks,
                   num_q_heads=b.num_q_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                   dtype=b.dtype, scale=b.scale, num_kv_splits=kw.pop("num_kv_splits", b.num_kv_splits),
                   tree_parent=kw.pop("tree_parent", b.tree_parent), cascade=kw.pop("cascade", 0), **kw)


def check_plan(b, p, num_cus=0):
    t = p.tables()
    grp = b.num_q_heads // b.num_kv_heads
    rs, rp = R.row_tables(b.q_len, b.q_start)
    assert np.array_equal(t["row_seq"], rs) and np.array_equal(t["row_pos"], rp)
    tree = R.row_tree_masks(b.q_len, b.tree_parent) is not None
    ns = R.num_splits(b.q_len, b.q_start, b.num_kv_heads, grp, b.num_kv_splits, num_cus, b.dtype, tree)
    assert np.array_equal(t["num_splits"], ns)
    bounds = R.seq_bounds(b.q_len, b.q_start, b.num_kv_heads, grp, ns, num_cus, b.dtype, b.num_kv_splits)
    lo, hi = R.split_ranges(b.q_len, b.q_start, ns, bounds)
    assert np.array_equal(t["split_begin"], lo) and np.array_equal(t["split_end"], hi)
    got = {tuple(int(x) for x in it[:7]) for it in t["items"]}
    assert len(got) == t["items"].shape[0], "duplicate tasks"
    assert got == R.expected_tasks(b.q_len, b.q_start, b.num_kv_heads, grp, ns, bounds)
    R.check_coverage(t["items"], b.q_len, b.q_start, b.num_kv_heads)
    check_records(b, t)
    return t


def check_records(b, t):
    """Direct tasks write each (row, head) once; split (row, head) pairs have one
    merge row whose records are exactly the parts its tasks write."""
    grp = b.num_q_heads // b.num_kv_heads
    items, merge = t["items"], t["merge_rows"]
    direct, recs = {}, {}
    for it in items:
        seq, g, r0, ntok, p0, lo, hi, part = (int(x) for x in it)
        for m in range(ntok * grp):
            key = (r0 + m // grp, g * grp + m % grp)
            if part < 0:
                direct[key] = direct.get(key, 0) + 1
            else:
                recs.setdefault(key, []).append(part + m)
    assert all(v == 1 for v in direct.values())
    seen = set()
    for rec0, stride, nparts, row, qh in merge:
        key = (int(row), int(qh))
        assert key not in direct and key not in seen
        seen.add(key)
        assert sorted(recs[key]) == [int(rec0) + p * int(stride) for p in range(int(nparts))]
    assert seen == set(recs)
    assert len(direct) + len(seen) == t["row_seq"].shape[0] * b.num_q_heads
    allrec = [r for v in recs.values() for r in v]
    assert len(set(allrec)) == len(allrec) and (not allrec or max(allrec) < t["num_part_records"])
    # classes are contiguous ranges whose tasks fit the class's row count
    cb, cr = t["class_begin"], t["class_rows"]
    assert cb[0] == 0 and cb[-1] == items.shape[0]
    for c in range(cr.shape[0]):
        rows = items[cb[c]:cb[c + 1], 3] * grp
        assert (rows <= cr[c]).all()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 7])
def test_plan_tables_match_replica(cfg):
    b = wl.config(cfg, values=False)
    check_plan(b, make_plan(b))


@pytest.mark.parametrize("splits", [0, 1, 3, 16])
@pytest.mark.parametrize("seed", range(4))
def test_plan_random_small_batches(splits, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    for hq, hkv in ((4, 4), (8, 2), (32, 8), (64, 1), (12, 4)):
        specs = []
        for _ in range(int(rng.integers(1, 9))):
            n = int(rng.integers(1, 300))
            ql = int(rng.integers(0, min(n, 70) + 1))
            qs = int(rng.integers(0, n - ql + 1))
            specs.append(dict(q_len=ql, seq_len=n, q_start=qs))
        b = wl.custom(specs, hq=hq, hkv=hkv, d=128, seed=seed, num_kv_splits=splits, values=False)
        for cus in (0, 3, 80):
            check_plan(b, make_plan(b, num_cus=cus), num_cus=cus)


def test_shuffle_changes_order_not_content():
    b = wl.config(4, values=False)
    a = make_plan(b).tables()
    s = make_plan(b, work_shuffle_seed=1234).tables()
    assert not np.array_equal(a["items"], s["items"])
    assert sorted(map(tuple, a["items"][:, :7].tolist())) == sorted(map(tuple, s["items"][:, :7].tolist()))
    check_plan(b, make_plan(b, work_shuffle_seed=1234))


def _xcd_of(kv_head, seq, hkv, xcds=8):
    """The XCD a task's kv head (and sequence) is meant for."""
    if hkv >= xcds:
        return kv_head % xcds
    rep = -(-xcds // hkv)
    return (kv_head * rep + seq % rep) % xcds


@pytest.mark.parametrize("cfg", [3, 4])
def test_dispatch_order_is_xcd_aware_and_cost_descending(cfg):
    """Workgroup slot i runs on XCD i % 8; every task of a kv head lands on that
    head's XCD, except where a workgroup is topped up from another XCD at the
    end of a queue (at most one workgroup per XCD here, since these workloads
    give every kv head the same number of tasks), and each XCD's own tasks come
    in non-increasing cost."""
    b = wl.config(cfg, values=False)
    t = make_plan(b).tables()
    it = t["items"]
    for c in range(t["class_rows"].shape[0]):
        cls = it[t["class_begin"][c]:t["class_begin"][c + 1]]
        per_wg = 4 if t["class_rows"][c] <= 64 else 1
        slot_xcd = (np.arange(cls.shape[0]) // per_wg) % 8
        want = np.array([_xcd_of(int(h), int(s_), b.num_kv_heads) for s_, h in zip(cls[:, 0], cls[:, 1])])
        assert (slot_xcd != want).sum() <= 8 * per_wg
        blk = -(-(cls[:, 6] - cls[:, 5]) // 16)
        for x in range(8):
            assert (np.diff(blk[want == x]) <= 0).all()


@pytest.mark.parametrize("cfg,num_cus", [(2, 0), (2, 64)])
def test_equal_work_decode_slots(cfg, num_cus):
    """Pure decode plans: wave w runs the tasks of slot w, all of one kv head,
    on that head's XCD (topped-up workgroups aside), each slot one piece of L
    blocks of the sequences laid end to end (the last piece of a head may be
    shorter), its tasks in sequence order and back to back."""
    b = wl.config(cfg, values=False)
    t = make_plan(b, num_cus=num_cus).tables()
    assert t["class_rows"].tolist() == [16]
    sb, it = t["slot_begin"], t["items"]
    assert sb.size > 1 and sb[0] == 0 and sb[-1] == it.shape[0] and (np.diff(sb) > 0).all()
    nblk = -(-(np.asarray(b.q_start) + np.asarray(b.q_len)) // 16)
    start = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    total = int(nblk.sum())
    per_head = max(1, (num_cus or 256) * 3 // b.num_kv_heads)
    L = max(16, -(-total // per_head))
    off_xcd = 0
    pieces = set()
    for w in range(sb.size - 1):
        tk = it[sb[w]:sb[w + 1]]
        g = set(tk[:, 1].tolist())
        assert len(g) == 1
        g = g.pop()
        off_xcd += (w // 4) % 8 != g % 8
        a = start[tk[:, 0]] + tk[:, 5] // 16                  # first block, in the concatenation
        e = start[tk[:, 0]] + -(-tk[:, 6] // 16)
        assert (a[1:] == e[:-1]).all() and (np.diff(tk[:, 0]) > 0).all()
        j = a[0] // L
        assert a[0] == j * L and (e[-1] == (j + 1) * L or e[-1] == total)
        pieces.add((g, int(j)))
    assert len(pieces) == sb.size - 1 == b.num_kv_heads * -(-total // L)
    assert off_xcd <= 8 * 4
    check_plan(b, make_plan(b, num_cus=num_cus), num_cus=num_cus)


def test_equal_work_only_for_pure_auto_split_bf16_decode():
    # explicit splits (the long-decode workload asks for 16), f32, or a verify row: one task per wave
    for b in (wl.config(5, values=False), wl.config(1, values=False),
              wl.custom([dict(q_len=1, seq_len=300), dict(q_len=5, seq_len=90)], hq=8, hkv=2, d=128,
                        values=False)):
        assert make_plan(b).tables()["slot_begin"].size == 0
    b = wl.custom([dict(q_len=1, seq_len=n) for n in (300, 17, 1000)], hq=8, hkv=2, d=128, values=False)
    assert make_plan(b).tables()["slot_begin"].size > 0
    # verify drafts alone (20 rows: the 32-row class) get the plan too
    b = wl.custom([dict(q_len=5, seq_len=n) for n in (300, 17, 1000)], hq=8, hkv=2, d=128, values=False)
    assert make_plan(b).tables()["slot_begin"].size > 0


def test_equal_work_verify_slots():
    """A batch of verify drafts only (32-row tasks): 4 waves per CU, each a
    run of pieces of L blocks of one kv head, like the decode plan."""
    rng = np.random.default_rng(3)
    b = wl.custom([dict(q_len=5, seq_len=int(n)) for n in rng.integers(6, 4000, 32)], hq=32, hkv=8, d=128,
                  seed=4, values=False)
    t = make_plan(b).tables()
    assert t["class_rows"].tolist() == [32]
    sb, it = t["slot_begin"], t["items"]
    nblk = -(-(np.asarray(b.q_start) + np.asarray(b.q_len)) // 16)
    start = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    total = int(nblk.sum())
    L = max(16, -(-total // max(1, 256 * 4 // b.num_kv_heads)))
    assert sb.size - 1 == b.num_kv_heads * -(-total // L)
    for w in range(sb.size - 1):
        tk = it[sb[w]:sb[w + 1]]
        assert len(set(tk[:, 1].tolist())) == 1
        a = start[tk[:, 0]] + tk[:, 5] // 16
        e = start[tk[:, 0]] + -(-tk[:, 6] // 16)
        assert (a[1:] == e[:-1]).all() and a[0] % L == 0 and (e[-1] % L == 0 or e[-1] == total)
    check_plan(b, make_plan(b))


def test_dispatch_order_with_few_kv_heads_is_a_permutation():
    b = wl.custom([dict(q_len=1, seq_len=n) for n in (40, 300, 77, 1000, 5)], hq=8, hkv=2, d=128)
    t = make_plan(b).tables()
    it = t["items"]
    # two kv heads: each spreads over 4 XCDs by sequence; the list still holds every task once
    u = make_plan(b, work_shuffle_seed=99).tables()["items"]
    assert sorted(map(tuple, it[:, :7].tolist())) == sorted(map(tuple, u[:, :7].tolist()))
    first = it[: min(8 * 4, it.shape[0])]
    xs = {_xcd_of(int(h), int(s_), 2) for s_, h in zip(first[:, 0], first[:, 1])}
    assert len(xs) > 2  # more than one XCD per kv head is used


def test_workspace_bytes():
    b = wl.config(5, values=False)
    p = make_plan(b)
    t = p.tables()
    assert p.workspace_bytes >= t["num_part_records"] * (128 + 1) * 4 + t["items"].shape[0] * 32
    assert p.workspace_bytes % 256 == 0


def _desc_kwargs(b):
    return dict(num_pool_blocks=b.num_pool_blocks, num_q_heads=b.num_q_heads,
                num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, dtype=b.dtype, scale=b.scale)


def test_error_paths():
    b = wl.custom([dict(q_len=2, seq_len=40, q_start=38), dict(q_len=1, seq_len=17)],
                  hq=4, hkv=2, d=64, values=False)
    kw = _desc_kwargs(b)

    def err(status, **over):
        args = dict(q_len=b.q_len, seq_len=b.seq_len, q_start=b.q_start, block_table=b.block_table)
        k2 = dict(kw)
        for k, v in over.items():
            (args if k in args else k2)[k] = v
        with pytest.raises(pm.PmattnError) as e:
            pm.plan(args["q_len"], args["seq_len"], args["q_start"], args["block_table"], **k2)
        assert e.value.status == status, str(e.value)
        return str(e.value)

    INV, UNS = _lib.E_INVALID, _lib.E_UNSUPPORTED
    assert "q_start + q_len > seq_len" in err(INV, q_start=np.array([39, 16]))
    err(INV, q_len=np.array([-1, 1]))
    bad = b.block_table.copy()
    bad[0, 1] = b.num_pool_blocks
    assert "block id" in err(INV, block_table=bad)
    bad[0, 1] = -1
    err(INV, block_table=bad)
    err(INV, block_table=b.block_table[:, :2])           # stride < ceil(40/16)
    err(INV, num_q_heads=6, num_kv_heads=4)
    err(INV, scale=0.0)
    err(INV, scale=float("nan"))
    err(INV, num_kv_splits=257)
    err(INV, num_kv_splits=-1)
    err(UNS, head_dim=96)
    err(UNS, num_q_heads=130, num_kv_heads=1)
    # block size is fixed at 16 by the binding; check the C check directly
    lib = _lib.load()
    d = _lib.PlanDesc(num_seqs=0, block_size=8, num_q_heads=1, num_kv_heads=1, head_dim=64, dtype=0,
                      scale=1.0)
    h = ctypes.c_void_p()
    assert lib.pmattn_plan(ctypes.byref(d), ctypes.byref(h)) == UNS
    assert b"block_size" in lib.pmattn_last_error()
    d = _lib.PlanDesc(num_seqs=0, block_size=16, num_q_heads=1, num_kv_heads=1, head_dim=64,
                      dtype=7, scale=1.0)
    assert lib.pmattn_plan(ctypes.byref(d), ctypes.byref(h)) == UNS
    d = _lib.PlanDesc(num_seqs=2, block_size=16, num_q_heads=1, num_kv_heads=1, head_dim=64,
                      dtype=0, scale=1.0)                  # null arrays
    assert lib.pmattn_plan(ctypes.byref(d), ctypes.byref(h)) == INV
    assert lib.pmattn_plan(None, ctypes.byref(h)) == INV


@pytest.mark.parametrize("seed", range(6))
def test_tree_masks_match_replica(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    seqs = []
    for k in range(int(rng.integers(1, 6))):
        kind = int(rng.integers(0, 4))
        ql = int(rng.integers(1, 65))
        qs = int(rng.integers(0, 200))
        spec = dict(q_len=ql, seq_len=qs + ql + int(rng.integers(0, 20)), q_start=qs)
        if kind == 0:
            spec["tree"] = wl.random_tree(ql, seed * 10 + k)
        elif kind == 1:
            spec["tree"] = wl.random_tree(ql, seed * 10 + k, max_depth=int(rng.integers(1, 5)))
        elif kind == 2:
            spec["q_len"] = ql = int(rng.integers(1, 200))      # causal, may exceed 64 rows
            spec["seq_len"] = qs + ql
        seqs.append(spec)
    seqs.append(dict(q_len=6, seq_len=40, tree=[-1, 0, 1, 1, 0, -1]))
    b = wl.custom(seqs, hq=8, hkv=2, d=64, values=False)
    p = make_plan(b)
    check_plan(b, p)
    t = p.tables()
    want = R.row_tree_masks(b.q_len, b.tree_parent)
    assert want is not None and t["row_tree_mask"] is not None
    assert np.array_equal(t["row_tree_mask"], want)
    # the same batch declared causal (or with chain parents) carries no masks
    assert make_plan(b, tree_parent=None).tables()["row_tree_mask"] is None
    chain = np.concatenate([np.arange(-1, int(q) - 1) for q in b.q_len])
    assert make_plan(b, tree_parent=chain).tables()["row_tree_mask"] is None


def test_tree_errors():
    b = wl.custom([dict(q_len=3, seq_len=40), dict(q_len=70, seq_len=90)], hq=4, hkv=2, d=64,
                  values=False)
    kw = _desc_kwargs(b)
    ok = np.concatenate([[-1, 0, 0], np.arange(-1, 69)])
    pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, tree_parent=ok, **kw)  # 70-row chain
    for bad_first, status, text in (([-1, 1, 0], _lib.E_INVALID, "tree_parent"),
                                    ([-2, 0, 0], _lib.E_INVALID, "tree_parent"),
                                    ([0, 0, 0], _lib.E_INVALID, "tree_parent")):
        tp = ok.copy()
        tp[:3] = bad_first
        with pytest.raises(pm.PmattnError) as e:
            pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, tree_parent=tp, **kw)
        assert e.value.status == status and text in str(e.value)
    tp = ok.copy()
    tp[3 + 5] = 2                      # the 70-row sequence stops being a chain
    with pytest.raises(pm.PmattnError) as e:
        pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, tree_parent=tp, **kw)
    assert e.value.status == _lib.E_UNSUPPORTED and "64" in str(e.value)
    with pytest.raises(ValueError):
        pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, tree_parent=ok[:-1], **kw)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_append_units_match_replica(cfg):
    b = wl.config(cfg, values=False)
    t = make_plan(b).tables()
    want = R.append_units(b.q_len, b.q_start)
    assert np.array_equal(t["append_units"], want)
    # the units cover every query row exactly once, within one block each
    assert int(want[:, 2].sum()) == b.num_rows and (want[:, 2] + want[:, 4] <= 16).all()


def _append_status(p):
    """pmattn_kv_append's verdict on a plan, with every pointer NULL: a plan that
    writes shared slots is refused before anything else is looked at."""
    lib = _lib.load()
    st = lib.pmattn_kv_append(p.handle, None, None, None, None, None, None, 0, None)
    return st, lib.pmattn_last_error().decode()


def test_append_refuses_shared_target_slots():
    # two sequences share block "a" (their first 16 tokens)
    b = wl.custom([dict(q_len=1, seq_len=20, nodes=["a"]), dict(q_len=1, seq_len=30, nodes=["a"])],
                  node_blocks={"a": 1}, hq=4, hkv=2, d=64, values=False)
    st, msg = _append_status(make_plan(b))
    assert st == _lib.E_INVALID and "non-NULL" in msg          # private targets: only NULLs are wrong
    # sequence 0 appends at position 10, inside the shared block that sequence 1 sees whole
    b2 = b.replace(q_start=np.array([10, 29], np.int32), seq_len=np.array([11, 30], np.int32))
    st, msg = _append_status(make_plan(b2))
    assert st == _lib.E_INVALID and "copy the block first" in msg
    # sequence 1 appends at position 7 of the shared block, which sequence 0 sees
    b3 = b.replace(q_start=np.array([10, 7], np.int32), seq_len=np.array([11, 8], np.int32))
    st, msg = _append_status(make_plan(b3))
    assert st == _lib.E_INVALID and "copy the block first" in msg
    # a sharer without query rows reads nothing, so the append is allowed
    b4 = b.replace(q_start=np.array([10, 3], np.int32), seq_len=np.array([11, 4], np.int32),
                   q_len=np.array([1, 0], np.int32))
    st, msg = _append_status(make_plan(b4))
    assert "non-NULL" in msg
    # two rows writing one slot
    b5 = b.replace(q_start=np.array([5, 5], np.int32), seq_len=np.array([6, 6], np.int32))
    st, msg = _append_status(make_plan(b5))
    assert st == _lib.E_INVALID and "same pool slot" in msg


def _check_cascade_plan(b, t, num_kv_splits=0, num_cus=0, mode=1):
    grp = b.num_q_heads // b.num_kv_heads
    rep = R.plan_units(b.q_len, b.q_start, b.block_table, b.num_kv_heads, grp, num_kv_splits, num_cus,
                       cascade=mode, dtype=b.dtype, tree=R.row_tree_masks(b.q_len, b.tree_parent) is not None)
    units = rep["units"]
    nb = b.num_seqs
    virt = units[nb:]
    assert t["cascade"]["lo"].tolist() == [u["lo"] for u in virt]
    assert t["cascade"]["hi"].tolist() == [u["hi"] for u in virt]
    assert t["cascade"]["seq"].tolist() == [u["seq"] for u in virt]
    assert t["cascade"]["row_begin"].tolist() == [u["row0"] for u in virt]
    assert t["cascade"]["rows"].tolist() == [u["rows"] for u in virt]
    assert t["cascade"]["splits"].tolist() == [u["splits"] for u in virt]
    assert np.array_equal(t["virtual_row_src"], rep["vrow_src"])
    assert t["num_splits"].tolist() == [u["splits"] for u in units[:nb]]
    lo = [x for u in units[:nb] for x, _ in u["bounds"]]
    hi = [x for u in units[:nb] for _, x in u["bounds"]]
    assert t["split_begin"].tolist() == lo and t["split_end"].tolist() == hi
    R.check_coverage_cascade(t["items"], t["class_cascade"], t["class_begin"], t["virtual_row_src"],
                             b.q_len, b.q_start, b.num_kv_heads)
    # every output (row, head) is written once directly or merged once, and a
    # merge row's records are exactly those its tasks write
    written = {}
    for c in range(len(t["class_rows"])):
        for it in t["items"][t["class_begin"][c]:t["class_begin"][c + 1]]:
            seq, kvh, r0, nt, p0, lo_, hi_, part = (int(x) for x in it[:8])
            for tt in range(nt):
                row = int(t["virtual_row_src"][r0 + tt]) if t["class_cascade"][c] else r0 + tt
                for i in range(grp):
                    key = (row, kvh * grp + i)
                    written.setdefault(key, []).append(None if part < 0 else part + tt * grp + i)
    merged = set()
    for rec0, stride, npart, row, qh in t["merge_rows"]:
        recs = (t["rec_index"][rec0:rec0 + npart].tolist() if stride < 0
                else [rec0 + k * stride for k in range(npart)])
        assert sorted(recs) == sorted(written[(int(row), int(qh))]), (row, qh)
        merged.add((int(row), int(qh)))
    for key, recs in written.items():
        assert (None in recs) == (key not in merged) and (len(recs) == 1 or key in merged)


@pytest.mark.parametrize("cfg", [1, 4, 5, 7])
@pytest.mark.parametrize("mode", [1, 2])
def test_cascade_plans_match_replica(cfg, mode):
    b = wl.config(cfg, values=False)
    t = make_plan(b, cascade=mode).tables()
    # mode 1 groups every shared run; the automatic mode leaves out the pairs
    # of the long-decode batch and the tiny batch, and the mixed batch's few
    # groups (they spare 7% of its keys)
    assert (t["cascade"]["lo"].shape[0] > 0) == (mode == 1 or cfg == 7)
    _check_cascade_plan(b, t, b.num_kv_splits, mode=mode)


@pytest.mark.parametrize("own, grouped", [(100, True), (8000, False)])
def test_cascade_auto_needs_a_quarter_of_the_keys_spared(own, grouped):
    # ten decode rows on one 64-block shared run: with 100 own tokens each the
    # group spares 9 x 1024 of 11,240 keys (82%), with 8,000 only 10%
    seqs = [dict(q_len=1, seq_len=1024 + own, nodes=[("n", 0)]) for _ in range(10)]
    b = wl.custom(seqs, node_blocks={("n", 0): 64}, hq=8, hkv=2, d=64, values=False)
    t = make_plan(b, cascade=2).tables()
    assert (t["cascade"]["lo"].shape[0] > 0) == grouped
    _check_cascade_plan(b, t, 0, mode=2)
    assert make_plan(b, cascade=1).tables()["cascade"]["lo"].shape[0] == 1

@pytest.mark.parametrize("seed", range(5))
def test_cascade_random_batches(seed):
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    nodes = {("n", k): int(rng.integers(1, 6)) for k in range(6)}
    seqs = []
    for _ in range(int(rng.integers(2, 14))):
        path = [("n", 0)] + [("n", int(k)) for k in sorted(rng.choice(np.arange(1, 6), size=int(rng.integers(0, 3)),
                                                                       replace=False))]
        shared = sum(nodes[n] for n in path) * 16
        ql = int(rng.choice([1, 1, 2, 5, 20, 40]))
        extra = int(rng.integers(0, 50))
        seqs.append(dict(q_len=ql, seq_len=shared + extra + ql, nodes=path))
    b = wl.custom(seqs, node_blocks=nodes, hq=8, hkv=2, d=64, values=False)
    for splits in (0, 3):
        bb = b.replace(num_kv_splits=splits)
        _check_cascade_plan(bb, make_plan(bb, cascade=1).tables(), splits)
        _check_cascade_plan(bb, make_plan(bb, cascade=2).tables(), splits, mode=2)
    # with the cascade off, the unit rules reproduce the plain tables
    rep = R.plan_units(b.q_len, b.q_start, b.block_table, b.num_kv_heads, 4)
    assert [u["splits"] for u in rep["units"]] == R.num_splits(b.q_len, b.q_start, b.num_kv_heads, 4).tolist()


def test_unused_table_entries_are_not_validated():
    # entries past the visible blocks may be anything (here -1); rows of length 0 read nothing
    b = wl.custom([dict(q_len=1, seq_len=20, q_start=5), dict(q_len=0, seq_len=33)], hq=2, hkv=1,
                  d=64, values=False)
    bt = b.block_table.copy()
    bt[0, 1] = -7        # block 1 holds keys 16..19, invisible to the row at position 5
    bt[1, :] = 10 ** 6   # sequence without rows
    p = pm.plan(b.q_len, b.seq_len, b.q_start, bt, **_desc_kwargs(b))
    t = p.tables()
    assert t["num_splits"].tolist() == [1, 0] and t["items"].shape[0] == 1


def test_empty_batch():
    p = pm.plan(np.zeros(0), np.zeros(0), np.zeros(0), np.zeros((0, 1)), num_pool_blocks=0,
                num_q_heads=1, num_kv_heads=1, head_dim=64, dtype="bf16", scale=1.0)
    t = p.tables()
    assert t["items"].shape[0] == 0 and t["row_seq"].shape[0] == 0 and p.workspace_bytes >= 256


def test_library_exports_every_declared_symbol():
    import glob
    declared = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        declared |= set(re.findall(r"\b(pmattn_[a-z_]+)\s*\(", open(h).read()))
    declared -= {"pmattn_plan_s"}
    assert {"pmattn_plan", "pmattn_forward", "pmattn_merge_lse", "pmattn_kv_append",
            "pmattn_radix_admit", "pmattn_copy_blocks"} <= declared
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == {n for n, _, _ in _lib.SIGNATURES}
    assert pm.version() == "0.1.0"


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_streaming_classes_match_replica(cfg, mode):
    """The per-class non-temporal flag equals the replica's reading of the
    exported work list: no block of the class is read for two sequences."""
    b = wl.config(cfg, values=False)
    t = make_plan(b, cascade=mode).tables()
    tasks, want = R.streaming_tasks(t["items"], t["class_begin"], t["class_cascade"], b.block_table)
    assert t["item_stream"].tolist() == tasks.tolist()
    assert t["class_stream"].tolist() == want.tolist()
    if cfg == 2:
        assert want.tolist() == [1]           # private blocks only
    if cfg == 5 and mode != 1:
        # turns 1-3 shared in pairs, turn 4 private: partitions 12-15 stream
        assert want.tolist() == [2]
        it = t["items"]
        assert (tasks == (it[:, 5] >= 24576)).all()
    if cfg == 7 and mode:
        # the cascade reads the prompt once; the members' own ranges are private
        assert [s for s, c in zip(want, t["class_cascade"]) if not c] == [1]


@pytest.mark.parametrize("seed", range(4))
def test_streaming_classes_random_batches(seed):
    rng = np.random.Generator(np.random.PCG64(500 + seed))
    nodes = {("n", k): int(rng.integers(1, 5)) for k in range(4)}
    seqs = []
    for _ in range(int(rng.integers(2, 12))):
        path = [("n", int(k)) for k in sorted(rng.choice(4, size=int(rng.integers(0, 3)), replace=False))]
        shared = sum(nodes[n] for n in path) * 16
        ql = int(rng.choice([1, 1, 3, 5, 20, 70]))
        seqs.append(dict(q_len=ql, seq_len=shared + int(rng.integers(0, 60)) + ql, nodes=path))
    b = wl.custom(seqs, node_blocks=nodes, hq=8, hkv=2, d=64, values=False)
    for mode in (0, 1, 2):
        for splits in (0, 3):
            bb = b.replace(num_kv_splits=splits)
            t = make_plan(bb, cascade=mode).tables()
            tasks, want = R.streaming_tasks(t["items"], t["class_begin"], t["class_cascade"], bb.block_table)
            assert t["item_stream"].tolist() == tasks.tolist()
            assert t["class_stream"].tolist() == want.tolist()


def _check_mixed_table(t):
    """The mixed-batch table runs every item exactly once: workgroup entries
    name items of classes above 32 rows, bundle slots items of 16- and 32-row
    classes (a bundle holds one of the two), and each entry's cascade bit
    matches its item's class."""
    n = t["items"].shape[0]
    cls_of = np.zeros(n, np.int64)
    casc_of = np.zeros(n, np.int64)
    for c in range(len(t["class_rows"])):
        cls_of[t["class_begin"][c]:t["class_begin"][c + 1]] = t["class_rows"][c]
        casc_of[t["class_begin"][c]:t["class_begin"][c + 1]] = t["class_cascade"][c]
    seen = np.zeros(n, np.int64)
    bundles = t["mix_bundles"].reshape(-1, 4)
    used_bundles = np.zeros(bundles.shape[0], np.int64)
    for e in t["mix_table"]:
        if e & 1:
            used_bundles[e >> 2] += 1
            kinds = set()
            for s in bundles[e >> 2]:
                if s < 0:
                    continue
                seen[s >> 1] += 1
                kinds.add(int(cls_of[s >> 1]))
                assert cls_of[s >> 1] <= 32 and casc_of[s >> 1] == (s & 1)
            assert len(kinds) == 1
        else:
            i = e >> 2
            seen[i] += 1
            assert cls_of[i] > 32 and casc_of[i] == ((e >> 1) & 1)
    assert (seen == 1).all() and (used_bundles == 1).all()


@pytest.mark.parametrize("cfg,cascade", [(4, 0), (4, 1), (4, 2), (7, 1), (7, 2)])
def test_mixed_table_covers_every_item_once(cfg, cascade):
    """Configs 4 (prefill, verify and decode rows) and 7 (decode rows whose
    shared prompt the cascade turns into workgroup tasks)."""
    b = wl.config(cfg, values=False)
    t = make_plan(b, cascade=cascade).tables()
    assert t["mixed_kernel"] == 1
    _check_mixed_table(t)


def test_mixed_table_tiles_of_one_partition_together():
    """Shared-prompt cascade: on each XCD (table position mod 8) the virtual
    tiles of one prompt partition sit side by side, partitions in key order, so
    that the tiles reading the same keys start together."""
    b = wl.config(7, values=False)
    t = make_plan(b, cascade=2).tables()
    items, table = t["items"], t["mix_table"]
    for x in range(8):
        wg = [items[e >> 2] for e in table[x::8] if not e & 1]
        assert len(wg) > 8
        keys = [(int(it[0]), int(it[6] - it[5]), int(it[5])) for it in wg]  # (seq, keys, first key)
        for a, c in zip(keys, keys[1:]):
            if a[:2] == c[:2]:
                assert a[2] <= c[2]
        # the first partition's tiles lead: the same first key, different row tiles
        first = [it for it in wg if int(it[5]) == int(wg[0][5]) and int(it[6]) == int(wg[0][6])]
        assert len(first) >= 2 and len({int(it[2]) for it in first}) == len(first)
        assert all(int(it[5]) == int(wg[0][5]) for it in wg[:len(first)])


@pytest.mark.parametrize("seed", range(12))
def test_mixed_table_random_batches(seed):
    rng = np.random.Generator(np.random.PCG64(400 + seed))
    specs = []
    for _ in range(int(rng.integers(2, 9))):
        n = int(rng.integers(1, 900))
        ql = int(rng.choice([1, 1, 3, 5, 40, 150]))
        ql = min(ql, n)
        specs.append(dict(q_len=ql, seq_len=n, q_start=n - ql))
    specs.append(dict(q_len=1, seq_len=int(rng.integers(1, 500))))
    specs.append(dict(q_len=70, seq_len=300, q_start=230))
    b = wl.custom(specs, hq=8, hkv=int(rng.choice([1, 2, 8])), d=128, seed=seed, values=False,
                  num_kv_splits=int(rng.choice([0, 0, 3])))
    t = make_plan(b, cascade=int(rng.integers(0, 3)), work_shuffle_seed=int(rng.integers(0, 3))).tables()
    assert t["mixed_kernel"] == 1
    _check_mixed_table(t)
    for dt, tree in (("f32", None), ("bf16", "tree")):
        bb = b.replace(dtype=dt) if dt == "f32" else b
        kw = {}
        if tree:
            # stars of at most 64 rows, chains beyond (still a tree plan)
            kw["tree_parent"] = np.concatenate([[-1] + [0] * (q - 1) if q <= 64 else list(range(-1, q - 1))
                                                for q in b.q_len]).astype(np.int32)
        tt = make_plan(bb, **kw).tables()
        if dt == "f32" or tt["row_tree_mask"] is not None:   # fp32, or a real token tree
            assert tt["mixed_kernel"] == 0
