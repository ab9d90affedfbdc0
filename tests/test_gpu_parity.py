"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: bf16 inputs max-abs <= 2e-2 and mean-abs <= 2e-3 over every compared
output element (lse within 1e-3); fp32 inputs max-abs <= 1e-5. Invariants the
pages state (shared = private blocks, padding never affects the output) and
the race check (work-list order) must hold bit-exactly on the GPU.
"""
import zlib

import numpy as np
import pytest

import oracle
import prefix_shared_paged_pmattn_amd as pm
import workloads as wl
from gpu_helpers import compare, make_plan, note, oracle_all_rows, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _batch_cases():
    S = dict
    return {
        # decode rows, GQA 4, ragged lengths across block edges
        "decode-g4-d128": (dict(hq=8, hkv=2, d=128), [S(q_len=1, seq_len=n) for n in (1, 15, 16, 17, 33, 100, 513, 1000)], 0),
        "decode-g8-d128-split3": (dict(hq=16, hkv=2, d=128), [S(q_len=1, seq_len=n) for n in (2, 47, 300, 777)], 3),
        "decode-g4-d64": (dict(hq=8, hkv=2, d=64), [S(q_len=1, seq_len=n) for n in (5, 64, 65, 129, 400)], 0),
        "verify5-g4": (dict(hq=8, hkv=2, d=128), [S(q_len=5, seq_len=n) for n in (5, 21, 37, 300)], 0),
        # equal-work decode plans: a long sequence cut into many pieces (a
        # many-partition merge) beside sequences that share one piece; fewer
        # kv heads than XCDs; d = 64
        "decode-equal-work-long-and-short": (dict(hq=8, hkv=2, d=128),
                                             [S(q_len=1, seq_len=n) for n in (20000, 3, 17, 700, 1)], 0),
        "decode-equal-work-d64": (dict(hq=16, hkv=4, d=64), [S(q_len=1, seq_len=n) for n in (5000, 40, 333)], 0),
        # equal-work plans of 32-row (verify) tasks: a long draft context cut
        # into many pieces beside short ones; G = 8 at d = 64 (24 rows)
        "verify-equal-work-long-and-short": (dict(hq=8, hkv=2, d=128),
                                             [S(q_len=5, seq_len=n) for n in (12000, 6, 40, 700, 5)], 0),
        "verify-equal-work-g8-d64": (dict(hq=16, hkv=2, d=64), [S(q_len=3, seq_len=n) for n in (3000, 50, 333)], 0),
        "prefill-unaligned": (dict(hq=8, hkv=2, d=128), [S(q_len=37, seq_len=42, q_start=5), S(q_len=100, seq_len=100),
                                                         S(q_len=64, seq_len=264, q_start=200)], 0),
        "prefill-d64-split2": (dict(hq=4, hkv=1, d=64), [S(q_len=70, seq_len=90, q_start=20), S(q_len=16, seq_len=16)], 2),
        "mha-g1": (dict(hq=4, hkv=4, d=128), [S(q_len=20, seq_len=50, q_start=30), S(q_len=1, seq_len=80)], 0),
        "g2": (dict(hq=6, hkv=3, d=64), [S(q_len=9, seq_len=30, q_start=21), S(q_len=3, seq_len=3)], 0),
        "g16": (dict(hq=32, hkv=2, d=128), [S(q_len=5, seq_len=60, q_start=55), S(q_len=1, seq_len=19)], 0),
        "g32": (dict(hq=32, hkv=1, d=128), [S(q_len=3, seq_len=40, q_start=37), S(q_len=1, seq_len=33)], 0),
        "g64": (dict(hq=64, hkv=1, d=64), [S(q_len=2, seq_len=50, q_start=48), S(q_len=1, seq_len=7)], 0),
        "g12-ragged": (dict(hq=12, hkv=1, d=128), [S(q_len=11, seq_len=99, q_start=88)], 0),
        "empty-seqs-mixed": (dict(hq=8, hkv=2, d=128), [S(q_len=0, seq_len=10), S(q_len=3, seq_len=35),
                                                        S(q_len=0, seq_len=0), S(q_len=1, seq_len=64)], 0),
        "many-splits-empty-parts": (dict(hq=8, hkv=2, d=128), [S(q_len=1, seq_len=40), S(q_len=4, seq_len=200)], 64),
        "position-zero": (dict(hq=4, hkv=2, d=128), [S(q_len=1, seq_len=1, q_start=0), S(q_len=4, seq_len=4, q_start=0)], 0),
        "keys-beyond-last-query": (dict(hq=8, hkv=2, d=128), [S(q_len=3, seq_len=90, q_start=10)], 0),
        # workgroup (128-row) tasks: partial records, long MHA runs, d=64, tiny contexts
        "prefill-wg-splits": (dict(hq=8, hkv=2, d=128), [S(q_len=100, seq_len=300, q_start=200), S(q_len=65, seq_len=65)], 3),
        "prefill-mha-long": (dict(hq=2, hkv=2, d=128), [S(q_len=200, seq_len=260, q_start=60)], 0),
        "prefill-d64-g8": (dict(hq=16, hkv=2, d=64), [S(q_len=33, seq_len=50, q_start=17), S(q_len=9, seq_len=9)], 0),
        "prefill-wg-tail-in-first-chunk": (dict(hq=8, hkv=2, d=128), [S(q_len=20, seq_len=23, q_start=3)], 0),
        # workgroup tasks whose last waves hold few or no rows; a run of whole
        # tasks followed by a one-token tail; d = 64 with rows a multiple of 128
        "prefill-wg-sparse-waves": (dict(hq=8, hkv=1, d=128), [S(q_len=17, seq_len=300, q_start=283),
                                                                 S(q_len=33, seq_len=33)], 0),
        "prefill-wg-d64-exact": (dict(hq=4, hkv=1, d=64), [S(q_len=64, seq_len=100, q_start=36)], 2),
        # workgroup tasks of 1 to 5 chunks of 32 keys (the LDS ring's first
        # and last steps), ending on and just past chunk edges, at both head
        # dims, and with partitions that start inside the ring's reach
        "prefill-wg-ring-lengths": (dict(hq=8, hkv=2, d=128), [S(q_len=40, seq_len=n, q_start=n - 40)
                                                                for n in (40, 64, 65, 96, 97, 128, 129, 160)], 0),
        "prefill-wg-ring-d64-splits": (dict(hq=8, hkv=2, d=64), [S(q_len=36, seq_len=n, q_start=n - 36)
                                                                  for n in (36, 95, 161, 224)], 3),
        # wave and workgroup tasks in one plan (run concurrently on two streams)
        "mixed-classes": (dict(hq=8, hkv=2, d=128), [S(q_len=50, seq_len=300, q_start=250), S(q_len=1, seq_len=700),
                                                     S(q_len=5, seq_len=405), S(q_len=1, seq_len=33),
                                                     S(q_len=130, seq_len=130)], 0),
        # speculative token trees: one-wave classes 16/32/64, workgroup tasks,
        # partitions inside the tree, G = 8 at d = 64, star and chain shapes
        "tree-wave-classes": (dict(hq=8, hkv=2, d=128), [S(q_len=4, seq_len=300, tree=wl.random_tree(4, 1)),
                                                         S(q_len=8, seq_len=208, q_start=200, tree=wl.random_tree(8, 2)),
                                                         S(q_len=16, seq_len=516, q_start=500,
                                                           tree=wl.random_tree(16, 3, max_depth=4)),
                                                         S(q_len=1, seq_len=90), S(q_len=5, seq_len=77)], 0),
        "tree-workgroup": (dict(hq=8, hkv=2, d=128), [S(q_len=64, seq_len=1064, q_start=1000,
                                                        tree=wl.random_tree(64, 4, max_depth=6)),
                                                      S(q_len=40, seq_len=73, q_start=33, tree=wl.random_tree(40, 5))], 0),
        "tree-splits": (dict(hq=8, hkv=2, d=128), [S(q_len=12, seq_len=60, q_start=48, tree=wl.random_tree(12, 6)),
                                                   S(q_len=64, seq_len=80, q_start=16, tree=wl.random_tree(64, 7)),
                                                   S(q_len=3, seq_len=45, q_start=42, tree=[-1, -1, 1])], 5),
        "tree-g8-d64": (dict(hq=16, hkv=2, d=64), [S(q_len=8, seq_len=40, q_start=32, tree=[-1, 0, 0, 1, 1, 2, -1, 6]),
                                                   S(q_len=30, seq_len=130, q_start=100, tree=wl.random_tree(30, 8))], 0),
        "tree-star-chain-mixed": (dict(hq=8, hkv=2, d=128), [S(q_len=16, seq_len=116, q_start=100, tree=[-1] * 16),
                                                             S(q_len=10, seq_len=30, q_start=20, tree=list(range(-1, 9))),
                                                             S(q_len=60, seq_len=400, q_start=340), S(q_len=1, seq_len=500),
                                                             S(q_len=33, seq_len=1033, q_start=1000,
                                                               tree=wl.random_tree(33, 9, max_depth=3))], 0),
    }


CASES = _batch_cases()


@pytest.mark.parametrize("name", sorted(CASES))
def test_small_batches(name):
    shape, specs, splits = CASES[name]
    b = wl.custom(specs, seed=zlib.crc32(name.encode()) % 1000, num_kv_splits=splits, name=name, extra_blocks=2,
                  **shape)
    note(f"case {name}: rows={b.num_rows}")
    out, lse = run_gpu(b)
    compare(b, out, lse)


def test_config1_f32_plumbing():
    b = wl.config(1)
    out, lse = run_gpu(b)
    compare(b, out, lse)


def test_f32_token_tree():
    b = wl.custom([dict(q_len=9, seq_len=50, q_start=41, tree=wl.random_tree(9, 11)),
                   dict(q_len=1, seq_len=20), dict(q_len=20, seq_len=36, q_start=16, tree=wl.random_tree(20, 12))],
                  hq=4, hkv=2, d=64, dtype="f32", seed=5, num_kv_splits=4)
    out, lse = run_gpu(b)
    compare(b, out, lse)


def test_f32_splits_and_gqa():
    b = wl.custom([dict(q_len=3, seq_len=70, q_start=60), dict(q_len=1, seq_len=33)], hq=4, hkv=2,
                  d=128, dtype="f32", seed=3, num_kv_splits=3)
    out, lse = run_gpu(b)
    compare(b, out, lse)


def test_single_key_is_exact():
    """One visible key: p = 1 exactly, so the output is V_0 bit for bit."""
    b = wl.custom([dict(q_len=1, seq_len=1, q_start=0), dict(q_len=1, seq_len=17, q_start=0)],
                  hq=8, hkv=2, d=128, seed=4)
    out, lse = run_gpu(b)
    for s in range(2):
        for h in range(8):
            v0 = wl.bf16_bits_to_f32(b.v_pool[b.block_table[s, 0], h // 4, :, 0]).astype(np.float64)
            assert np.array_equal(out[s, h], v0)
    compare(b, out, lse)


def test_full_config2_decode():
    b = wl.config(2)
    note(f"config 2: {b.num_rows} rows, {b.num_pool_blocks} blocks")
    out, lse = run_gpu(b)
    compare(b, out, lse)


def test_full_config5_long_decode():
    b = wl.config(5)
    note(f"config 5: {b.num_rows} rows, {b.num_pool_blocks} blocks, splits {b.num_kv_splits}")
    out, lse = run_gpu(b)
    compare(b, out, lse)


def test_full_config3_every_row():
    """The few-shot workload at full size (32,768 rows x 32 heads), every
    output element and lse against the oracle."""
    b = wl.config(3)
    note(f"config 3: {b.num_rows} rows, every row")
    out, lse = run_gpu(b)
    compare(b, out, lse, ref=oracle_all_rows(b))


@pytest.mark.parametrize("cascade", [2, 1])
def test_full_config4_every_row(cascade):
    """The mixed batch at full size, every output element: automatic cascade
    (as bench.py launches it; no groups here) and every shared run grouped
    (cascade tasks beside prefill, decode and verify tasks)."""
    b = wl.config(4)
    note(f"config 4 (cascade {cascade}): {b.num_rows} rows, every row")
    out, lse = run_gpu(b, cascade=cascade)
    compare(b, out, lse, ref=oracle_all_rows(b, key="config4"))


def test_full_config6_tree_verify_every_row():
    """The token-tree verify workload at full size, as bench.py launches it."""
    b = wl.config(6)
    note(f"config 6: {b.num_rows} rows, every row")
    out, lse = run_gpu(b)
    compare(b, out, lse, ref=oracle_all_rows(b))


def test_full_config7_shared_prompt_cascade_every_row():
    """The shared-prompt decode workload at full size with the automatic cascade."""
    b = wl.config(7)
    p = make_plan(b)
    assert p.tables()["cascade"]["lo"].shape[0] > 0, "the prompt should form a cascade group"
    note(f"config 7: {b.num_rows} rows, every row")
    out, lse = run_gpu(b)
    compare(b, out, lse, ref=oracle_all_rows(b))


def test_poison_in_invisible_slots_changes_nothing():
    b = wl.custom([dict(q_len=1, seq_len=37), dict(q_len=5, seq_len=50, q_start=41),
                   dict(q_len=20, seq_len=33, q_start=2), dict(q_len=3, seq_len=90, q_start=10)],
                  hq=8, hkv=2, d=128, seed=12, extra_blocks=3, num_kv_splits=2)
    ref_o, ref_l = run_gpu(b)
    for val in (float("nan"), 6e4, -6e4):
        o, l = run_gpu(wl.with_poison(b, val))
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l), val
    compare(b, ref_o, ref_l)


def test_work_order_does_not_change_bits():
    """Race check: any permutation of the work list gives bit-identical output."""
    b = wl.custom([dict(q_len=1, seq_len=n) for n in (100, 333, 517)] +
                  [dict(q_len=40, seq_len=300, q_start=260), dict(q_len=5, seq_len=80)],
                  hq=8, hkv=2, d=128, seed=5, num_kv_splits=3)
    dev = to_device(b)
    ref_o, ref_l = run_gpu(b, dev)
    for seed in (1, 2, 99):
        o, l = run_gpu(b, dev, work_shuffle_seed=seed)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)


def test_token_tree_order_and_poison_bitwise():
    """Token trees with split partitions: work-list shuffles and poison in slots
    no row can see leave every bit unchanged."""
    b = wl.custom([dict(q_len=20, seq_len=120, q_start=100, tree=wl.random_tree(20, 21)),
                   dict(q_len=64, seq_len=70, q_start=6, tree=wl.random_tree(64, 22, max_depth=5)),
                   dict(q_len=1, seq_len=77), dict(q_len=6, seq_len=50, q_start=40, tree=[-1, 0, 0, 1, 2, -1])],
                  hq=8, hkv=2, d=128, seed=23, extra_blocks=2, num_kv_splits=3)
    dev = to_device(b)
    ref_o, ref_l = run_gpu(b, dev)
    compare(b, ref_o, ref_l)
    for seed in (3, 7):
        o, l = run_gpu(b, dev, work_shuffle_seed=seed)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)
    o, l = run_gpu(wl.with_poison(b, float("nan")))
    assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)


def test_shared_blocks_equal_private_copies_bitwise():
    b = wl.custom([dict(q_len=3, seq_len=70, q_start=40, nodes=["a", "b"]), dict(q_len=1, seq_len=55, nodes=["a"]),
                   dict(q_len=2, seq_len=90, q_start=88, nodes=["a", "b"])],
                  node_blocks={"a": 2, "b": 1}, hq=8, hkv=2, d=128, seed=9)
    ref_o, ref_l = run_gpu(b)
    for other in (wl.private_copy(b), wl.relabel(b, 3)):
        o, l = run_gpu(other)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)
    compare(b, ref_o, ref_l)


def test_decode_row_matches_prefill_row():
    """Class independence on the GPU: a decode row equals the prefill row at the
    same position (within the bf16 bar; the tile shapes differ)."""
    pre = wl.custom([dict(q_len=6, seq_len=245, q_start=239)], hq=8, hkv=2, d=128, seed=21)
    po, pl = run_gpu(pre)
    for t in (0, 3, 5):
        dec = pre.replace(q_len=np.array([1], np.int32), q_start=np.array([239 + t], np.int32),
                          seq_len=np.array([240 + t], np.int32), q=pre.q[t:t + 1])
        o, l = run_gpu(dec)
        assert np.abs(o[0] - po[t]).max() <= 1e-2 and np.abs(l[0] - pl[t]).max() <= 1e-4


def test_two_passes_equal_forward():
    import torch
    b = wl.custom([dict(q_len=1, seq_len=n) for n in (300, 700)] + [dict(q_len=9, seq_len=100)],
                  hq=8, hkv=2, d=128, seed=6, num_kv_splits=4)
    dev = to_device(b)
    ref_o, ref_l = run_gpu(b, dev)
    p = make_plan(b)
    out = torch.zeros((b.num_rows, 8, 128), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros((b.num_rows, 8), dtype=torch.float32, device="cuda:0")
    ws = pm.forward_tasks(p, dev["q"], dev["k"], dev["v"], dev["bt"], out, lse)
    pm.forward_merge(p, out, lse, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), ref_o) and np.array_equal(lse.cpu().numpy(), ref_l)
    # the same workspace, uploaded once by hand and reused as resident
    ws2 = torch.empty(p.workspace_bytes, dtype=torch.uint8, device="cuda:0")
    p.upload(ws2)
    for _ in range(2):
        out.zero_()
        pm.forward(p, dev["q"], dev["k"], dev["v"], dev["bt"], out, lse, workspace=ws2, resident=True)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), ref_o)


def test_empty_plan_launches_nothing():
    import torch
    b = wl.custom([dict(q_len=0, seq_len=30)], hq=4, hkv=2, d=128, seed=1)
    p = make_plan(b)
    out = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device="cuda:0")
    dev = to_device(b)
    pm.forward(p, dev["q"], dev["k"], dev["v"], dev["bt"], out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("P", [2, 5, 8, 9, 12, 13, 100])  # group kernel up to 12 partials (one batch up to 8), wave kernel above
def test_merge_lse_standalone(d, out_dtype, P):
    import torch
    rng = np.random.Generator(np.random.PCG64(d + P))
    rows, H = 7, 3
    po = rng.standard_normal((P, rows, H, d)).astype(np.float32)
    pl = (rng.standard_normal((P, rows, H)) * 3).astype(np.float32)
    pl[1, 2, :] = -np.inf            # an empty partition: its output slot is not read
    po[1, 2, :] = np.nan
    pl[P - 1, 5, :] = -np.inf        # an empty partition past the first 64
    po[P - 1, 5, :] = np.nan
    pl[:, 4, 1] = -np.inf            # a row with every partition empty
    po[:, 4, 1] = np.nan
    ref_o, ref_l = oracle.merge_partitions(po.astype(np.float64), pl.astype(np.float64))
    et = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full((rows, H, d), float("nan"), dtype=et, device="cuda:0")
    lse = torch.full((rows, H), float("nan"), dtype=torch.float32, device="cuda:0")
    pm.merge_lse(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), out, lse)
    torch.cuda.synchronize()
    go = out.float().cpu().numpy()
    gl = lse.cpu().numpy()
    tol = 8e-3 if out_dtype == "bf16" else 2e-6
    assert np.abs(go - ref_o).max() <= tol
    fin = np.isfinite(ref_l)
    assert np.abs(gl[fin] - ref_l[fin]).max() <= 2e-6
    assert np.array_equal(np.isneginf(gl), ~fin) and (go[4, 1] == 0).all()


def test_forward_rejects_mis_sized_tensors():
    import torch
    b = wl.custom([dict(q_len=2, seq_len=20)], hq=4, hkv=2, d=128, seed=1)
    p = make_plan(b)
    dev = to_device(b)
    out = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        pm.forward(p, dev["q"][:1], dev["k"], dev["v"], dev["bt"], out)
    with pytest.raises(ValueError):
        pm.forward(p, dev["q"], dev["k"][:1], dev["v"], dev["bt"], out)
    with pytest.raises(ValueError):
        pm.forward(p, dev["q"], dev["k"], dev["v"], dev["bt"], out.float())
    with pytest.raises(ValueError):
        pm.forward(p, dev["q"], dev["k"], dev["v"], dev["bt"], out,
                   workspace=torch.zeros(16, dtype=torch.uint8, device="cuda:0"))


def _cascade_cases():
    S = dict
    nb = {"a": 4, "b": 2, "c": 3, "d": 1}
    return {
        # decode rows over nested shared runs, plus prefill and private rows
        "nested-decode": (dict(hq=8, hkv=2, d=128), nb, 0, [
            S(q_len=1, seq_len=130, nodes=["a", "b"]), S(q_len=1, seq_len=101, nodes=["a", "b"]),
            S(q_len=1, seq_len=200, nodes=["a", "c"]), S(q_len=1, seq_len=97, nodes=["a"]),
            S(q_len=5, seq_len=150, nodes=["a", "c"]), S(q_len=40, seq_len=140, q_start=100, nodes=["a", "c"]),
            S(q_len=1, seq_len=300)]),
        "verify-trees-splits": (dict(hq=8, hkv=2, d=128), nb, 3, [
            S(q_len=6, seq_len=120, nodes=["a", "d"], tree=[-1, 0, 0, 1, 2, -1]),
            S(q_len=12, seq_len=90, nodes=["a", "d"], tree=wl.random_tree(12, 4)),
            S(q_len=1, seq_len=77, nodes=["a"]), S(q_len=1, seq_len=66, nodes=["a", "d"])]),
        "g8-d64-many": (dict(hq=16, hkv=2, d=64), {"a": 6}, 0,
                        [S(q_len=1, seq_len=100 + 7 * i, nodes=["a"]) for i in range(20)]),
        "f32": (dict(hq=4, hkv=2, d=128, dtype="f32"), nb, 2, [
            S(q_len=1, seq_len=100, nodes=["a", "b"]), S(q_len=2, seq_len=113, nodes=["a", "b"]),
            S(q_len=1, seq_len=70, nodes=["a"])]),
        "wide-group": (dict(hq=8, hkv=2, d=128), {"a": 8}, 0,
                       [S(q_len=1, seq_len=129 + i, nodes=["a"]) for i in range(64)]),
    }


CASCADE = _cascade_cases()


@pytest.mark.parametrize("name", sorted(CASCADE))
def test_cascade_batches(name):
    shape, nodes, splits, specs = CASCADE[name]
    b = wl.custom(specs, node_blocks=nodes, seed=zlib.crc32(name.encode()) % 1000, num_kv_splits=splits,
                  name="cascade-" + name, extra_blocks=2, **shape)
    note(f"cascade case {name}: rows={b.num_rows}")
    p = make_plan(b, cascade=1)
    assert p.tables()["cascade"]["lo"].shape[0] > 0
    out, lse = run_gpu(b, cascade=1)
    compare(b, out, lse)


def test_cascade_full_config5_and_order():
    b = wl.config(5)
    dev = to_device(b)
    out, lse = run_gpu(b, dev, cascade=1)
    compare(b, out, lse)
    o2, l2 = run_gpu(b, dev, cascade=1, work_shuffle_seed=5)
    assert np.array_equal(o2, out) and np.array_equal(l2, lse)


def _share_mode_case(kind, d, extra):
    """Small batches whose one-wave class reads only shared blocks (stream
    mode 0), or shared and private ones (mode 2), alone, beside a workgroup
    task (the concurrent instance), or with token trees."""
    sh = [("n", 0)]
    if kind == "all-shared-decode":
        sp = [dict(q_len=1, seq_len=39 + i, nodes=sh) for i in range(4)]
    elif kind == "some-shared-decode":
        sp = [dict(q_len=1, seq_len=39 + i, nodes=sh) for i in range(3)] + [dict(q_len=1, seq_len=300 + i) for i in range(3)]
    elif kind == "all-shared-verify":
        sp = [dict(q_len=5, seq_len=41 + i, q_start=36 + i, nodes=sh) for i in range(4)]
    else:
        sp = ([dict(q_len=5, seq_len=41 + i, q_start=36 + i, nodes=sh) for i in range(3)] +
              [dict(q_len=5, seq_len=400 + i, q_start=395 + i) for i in range(2)])
    if extra == "beside-prefill":
        sp = sp + [dict(q_len=40, seq_len=90, q_start=50)]
    if extra == "tree":
        sp = [dict(s, tree=[-1] + [0] * (s["q_len"] - 1)) if s["q_len"] > 1 else s for s in sp]
        if all(s["q_len"] == 1 for s in sp):
            sp = sp + [dict(q_len=4, seq_len=60, q_start=56, tree=[-1, 0, 0, 1])]
    return wl.custom(sp, node_blocks={("n", 0): 2}, hq=8, hkv=2, d=d, seed=5, extra_blocks=2,
                     name=f"{kind}-d{d}-{extra}")


@pytest.mark.parametrize("extra", ["alone", "beside-prefill", "tree"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["all-shared-decode", "some-shared-decode", "all-shared-verify", "some-shared-verify"])
def test_stream_modes(kind, d, extra):
    """Cached (0) and per-task (2) K/V loads of the one-wave kernel give the
    oracle's result; the planner picks the intended mode."""
    b = _share_mode_case(kind, d, extra)
    t = make_plan(b).tables()
    wave = [s for r, s in zip(t["class_rows"], t["class_stream"]) if r <= 64]
    want = 0 if kind.startswith("all") and not (extra == "tree" and kind.endswith("decode")) else 2
    assert wave == [want], (t["class_rows"], t["class_stream"])
    note(f"stream mode case {b.name}: classes {t['class_rows'].tolist()} modes {t['class_stream'].tolist()}")
    out, lse = run_gpu(b)
    compare(b, out, lse)
