"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` takes an ``attend(batch, rows=None) -> (out, lse)`` callable
(the oracle, or a deliberately broken copy in the mutation test) and raises
``AssertionError`` when the callable disagrees with:

* closed forms (one key -> that key's value; equal scores -> mean of the values;
  two keys -> logistic weights; hand-derived fixtures under ``tests/golden/``),
* library routines on dense tensors (``torch.nn.functional.scaled_dot_product_attention``
  in float64 with an explicit boolean mask and its own GQA grouping;
  ``torch.logsumexp``), fed by K/V the test scatters into the pool itself,
* a 50-digit mpmath evaluation,
* invariants the pages state: shared prefix blocks = privately copied blocks
  and block relabeling (XY-Serve review, "Assumptions & free parameters",
  block-table/radix-tree item); one row-wise mask rule for prefill, decode and
  verify rows ("Editorial extensions"); output a convex combination of values.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _vals(b, arr):
    if b.dtype == "bf16":
        return wl.bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(b, x):
    x = np.asarray(x, dtype=np.float32)
    return wl.f32_to_bf16_bits(x) if b.dtype == "bf16" else x


def _dense_batch(seq_specs, hq, hkv, d, dtype, seed, shared_blocks=0):
    """Build dense per-sequence K/V first, then scatter them into a paged pool
    with randomly chosen physical blocks (optionally sharing the first
    ``shared_blocks`` blocks between all sequences). Returns the batch and the
    dense float64 K/V per sequence ([Hkv][n][d] each)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nseq = len(seq_specs)
    nblk = [-(-s["seq_len"] // 16) for s in seq_specs]
    total = shared_blocks + sum(n - shared_blocks for n in nblk) + 3   # 3 unused blocks
    perm = rng.permutation(total)
    shared_ids = perm[:shared_blocks]
    cur = shared_blocks
    stride = max(nblk)
    bt = np.full((nseq, stride), -1, np.int32)
    for s in range(nseq):
        own = perm[cur:cur + nblk[s] - shared_blocks]
        cur += nblk[s] - shared_blocks
        bt[s, :nblk[s]] = np.concatenate([shared_ids, own])
    k_pool = rng.standard_normal((total, hkv, 16, d)).astype(np.float32)
    v_pool = rng.standard_normal((total, hkv, d, 16)).astype(np.float32)
    dense_k, dense_v = [], []
    base_k = rng.standard_normal((max(s["seq_len"] for s in seq_specs), hkv, d)).astype(np.float32)
    base_v = rng.standard_normal((max(s["seq_len"] for s in seq_specs), hkv, d)).astype(np.float32)
    for s, spec in enumerate(seq_specs):
        n = spec["seq_len"]
        kd = rng.standard_normal((n, hkv, d)).astype(np.float32)
        vd = rng.standard_normal((n, hkv, d)).astype(np.float32)
        # tokens in the shared blocks are identical for every sequence
        ns = min(n, shared_blocks * 16)
        kd[:ns] = base_k[:ns]
        vd[:ns] = base_v[:ns]
        if dtype == "bf16":
            kd = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(kd))
            vd = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(vd))
        for t in range(n):
            blk, slot = bt[s, t // 16], t % 16
            for g in range(hkv):
                k_pool[blk, g, slot, :] = kd[t, g]
                v_pool[blk, g, :, slot] = vd[t, g]
        dense_k.append(kd.transpose(1, 0, 2).astype(np.float64))
        dense_v.append(vd.transpose(1, 0, 2).astype(np.float64))
    r = sum(s["q_len"] for s in seq_specs)
    q = rng.standard_normal((r, hq, d)).astype(np.float32)
    if dtype == "bf16":
        k_pool, v_pool, q = (wl.f32_to_bf16_bits(k_pool), wl.f32_to_bf16_bits(v_pool),
                             wl.f32_to_bf16_bits(q))
    k_pool = wl.k_pool_layout(k_pool, dtype)
    scale = float(np.float32(1.0 / math.sqrt(d) * (1.0 + 0.37 * (seed % 3))))
    b = wl.Batch(name="dense", q_len=np.array([s["q_len"] for s in seq_specs], np.int32),
                 seq_len=np.array([s["seq_len"] for s in seq_specs], np.int32),
                 q_start=np.array([s["q_start"] for s in seq_specs], np.int32), block_table=bt,
                 num_pool_blocks=total, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                 scale=scale, num_kv_splits=0, q=q, k_pool=k_pool, v_pool=v_pool)
    return b, dense_k, dense_v


def _sdpa_reference(b, dense_k, dense_v):
    """Dense reference through torch SDPA (float64, CPU, explicit bool mask, enable_gqa)."""
    out, lse = [], []
    row = 0
    qv = _vals(b, b.q)
    for s in range(b.num_seqs):
        ql, qs, n = int(b.q_len[s]), int(b.q_start[s]), int(b.seq_len[s])
        if ql == 0:
            continue
        qq = torch.from_numpy(qv[row:row + ql]).permute(1, 0, 2)[None]        # [1][Hq][ql][d]
        kk = torch.from_numpy(dense_k[s][:, :n])[None]                          # [1][Hkv][n][d]
        vv = torch.from_numpy(dense_v[s][:, :n])[None]
        pos = torch.arange(qs, qs + ql)[:, None]
        mask = torch.arange(n)[None, :] <= pos                                  # [ql][n]
        o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=b.scale,
                                           enable_gqa=True)
        grp = b.num_q_heads // b.num_kv_heads
        kx = kk.repeat_interleave(grp, dim=1)
        sc = (qq @ kx.transpose(-1, -2)) * b.scale
        sc = sc.masked_fill(~mask, float("-inf"))
        out.append(o[0].permute(1, 0, 2).numpy())
        lse.append(torch.logsumexp(sc, dim=-1)[0].permute(1, 0).numpy())
        row += ql
    return np.concatenate(out), np.concatenate(lse)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_single_key(attend):
    """A row at position 0 sees one key: output = that value row exactly; lse = its score."""
    b = wl.custom([dict(q_len=1, seq_len=1, q_start=0), dict(q_len=3, seq_len=19, q_start=0)],
                  hq=4, hkv=2, d=32, dtype="bf16", seed=11)
    out, lse = attend(b)
    bt = b.block_table
    qv = _vals(b, b.q)
    for row, s in ((0, 0), (1, 1)):
        for h in range(4):
            g = h // 2
            v0 = _vals(b, b.v_pool[bt[s, 0], g, :, 0])
            k0 = _vals(b, b.k_pool[bt[s, 0], g, :, 0, :].reshape(-1))
            assert np.array_equal(out[row, h], v0), "one visible key must give exactly V_0"
            s0 = b.scale * math.fsum(float(a) * float(c) for a, c in zip(qv[row, h], k0))
            assert abs(lse[row, h] - s0) <= 1e-12 * max(1.0, abs(s0))


def pin_equal_scores(attend):
    """q = 0 makes every score 0: output = mean of the visible values, lse = ln(pos+1)."""
    b = wl.custom([dict(q_len=4, seq_len=37, q_start=30), dict(q_len=1, seq_len=5, q_start=4)],
                  hq=2, hkv=1, d=16, dtype="f32", seed=5)
    b = b.replace(q=np.zeros_like(b.q))
    out, lse = attend(b)
    row = 0
    for s in range(2):
        for t in range(int(b.q_len[s])):
            pos = int(b.q_start[s]) + t
            vals = np.stack([_vals(b, b.v_pool[b.block_table[s, j // 16], 0, :, j % 16])
                             for j in range(pos + 1)])
            mean = np.array([math.fsum(vals[:, c]) / (pos + 1) for c in range(b.head_dim)])
            for h in range(2):
                assert np.allclose(out[row, h], mean, rtol=1e-14, atol=1e-15)
                assert abs(lse[row, h] - math.log(pos + 1)) < 1e-14
            row += 1


def pin_two_keys(attend):
    """Position 1 sees two keys: output = sigma(s0 - s1) V0 + sigma(s1 - s0) V1."""
    b = wl.custom([dict(q_len=2, seq_len=2, q_start=0)], hq=3, hkv=3, d=8, dtype="bf16", seed=7)
    out, lse = attend(b)
    qv = _vals(b, b.q)
    blk = b.block_table[0, 0]
    for h in range(3):
        k = [_vals(b, b.k_pool[blk, h, :, j, :].reshape(-1)) for j in (0, 1)]
        v = [_vals(b, b.v_pool[blk, h, :, j]) for j in (0, 1)]
        s = [b.scale * math.fsum(float(x) * float(y) for x, y in zip(qv[1, h], k[j])) for j in (0, 1)]
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        w1 = 1.0 / (1.0 + math.exp(s[0] - s[1]))
        assert np.allclose(out[1, h], w0 * v[0] + w1 * v[1], rtol=1e-13, atol=1e-14)
        assert abs(lse[1, h] - (max(s) + math.log1p(math.exp(min(s) - max(s))))) < 1e-13


def pin_golden(attend):
    """Hand-derived closed-form fixtures (tests/golden/*.json)."""
    for fn in sorted(os.listdir(GOLDEN)):
        if not fn.endswith(".json"):
            continue
        with open(os.path.join(GOLDEN, fn)) as f:
            fx = json.load(f)
        d = fx["head_dim"]
        keys = np.array(fx["keys"], np.float32)
        vals = np.array(fx["values"], np.float32)
        n = keys.shape[0]
        nb = -(-n // 16)
        k_pool = np.zeros((nb, 1, 16, d), np.float32)
        v_pool = np.zeros((nb, 1, d, 16), np.float32)
        for j in range(n):
            k_pool[j // 16, 0, j % 16] = keys[j]
            v_pool[j // 16, 0, :, j % 16] = vals[j]
        k_pool = wl.k_pool_layout(k_pool, "f32")
        b = wl.Batch(name=fn, q_len=np.array([1], np.int32), seq_len=np.array([n], np.int32),
                     q_start=np.array([n - 1], np.int32),
                     block_table=np.arange(nb, dtype=np.int32)[None], num_pool_blocks=nb,
                     num_q_heads=1, num_kv_heads=1, head_dim=d, dtype="f32",
                     scale=float(fx["scale"]), num_kv_splits=0,
                     q=np.array(fx["query"], np.float32)[None, None], k_pool=k_pool, v_pool=v_pool)
        out, lse = attend(b)
        assert np.allclose(out[0, 0], fx["expected_output"], rtol=0, atol=fx["tolerance"]), fn
        assert abs(lse[0, 0] - fx["expected_lse"]) <= fx["tolerance"], fn


def pin_brute_force_sdpa(attend):
    """Small exhaustive batches vs dense torch SDPA (fp64) on K/V scattered by the test."""
    shapes = [(1, 1), (2, 1), (4, 2), (6, 3)]
    dims = [1, 2, 4, 8, 24]
    cases = 0
    for ci, (hq, hkv) in enumerate(shapes):
        for di, d in enumerate(dims):
            seed = 100 + 10 * ci + di
            rng = np.random.Generator(np.random.PCG64(seed))
            specs = []
            for _ in range(int(rng.integers(1, 4))):
                n = int(rng.integers(1, 41))
                ql = int(rng.integers(1, min(5, n) + 1))
                qs = int(rng.integers(0, n - ql + 1))
                specs.append(dict(q_len=ql, seq_len=n, q_start=qs))
            shared = int(rng.integers(0, 1 + min(s["seq_len"] for s in specs) // 16))
            dtype = "bf16" if (ci + di) % 2 else "f32"
            b, dk, dv = _dense_batch(specs, hq, hkv, d, dtype, seed, shared_blocks=shared)
            ref_o, ref_l = _sdpa_reference(b, dk, dv)
            out, lse = attend(b)
            assert out.shape == ref_o.shape
            assert np.allclose(out, ref_o, rtol=1e-12, atol=1e-12), (hq, hkv, d)
            assert np.allclose(lse, ref_l, rtol=1e-12, atol=1e-12), (hq, hkv, d)
            cases += 1
    assert cases == len(shapes) * len(dims)


def pin_mpmath(attend):
    """A few rows evaluated with 50-digit arithmetic (mpmath), independent of numpy/BLAS."""
    import mpmath
    mpmath.mp.dps = 50
    specs = [dict(q_len=3, seq_len=35, q_start=32), dict(q_len=2, seq_len=18, q_start=7)]
    b, dk, dv = _dense_batch(specs, 4, 2, 8, "bf16", seed=3, shared_blocks=1)
    out, lse = attend(b)
    qv = _vals(b, b.q)
    row = 0
    for s, spec in enumerate(specs):
        for t in range(spec["q_len"]):
            pos = spec["q_start"] + t
            for h in range(4):
                g = h // 2
                sc = [mpmath.mpf(b.scale) * mpmath.fsum(mpmath.mpf(float(qv[row, h, c])) *
                                                        mpmath.mpf(float(dk[s][g, j, c]))
                                                        for c in range(8)) for j in range(pos + 1)]
                m = max(sc)
                w = [mpmath.e ** (x - m) for x in sc]
                tot = mpmath.fsum(w)
                for c in range(8):
                    o = mpmath.fsum(w[j] * mpmath.mpf(float(dv[s][g, j, c]))
                                    for j in range(pos + 1)) / tot
                    assert abs(float(o) - out[row, h, c]) <= 1e-13
                assert abs(float(m + mpmath.log(tot)) - lse[row, h]) <= 1e-13
            row += 1


def pin_shared_equals_private(attend):
    """Shared physical prefix blocks give the same result as private copies, and
    relabeling every physical block changes nothing."""
    b = wl.custom([dict(q_len=3, seq_len=70, q_start=40, nodes=["a", "b"]),
                   dict(q_len=1, seq_len=55, nodes=["a"]),
                   dict(q_len=2, seq_len=90, q_start=88, nodes=["a", "b"])],
                  node_blocks={"a": 2, "b": 1}, hq=4, hkv=2, d=16, dtype="bf16", seed=9)
    ref_o, ref_l = attend(b)
    for other in (wl.private_copy(b), wl.relabel(b, 4), wl.relabel(wl.private_copy(b), 8)):
        o, l = attend(other)
        assert np.allclose(o, ref_o, rtol=0, atol=1e-13)
        assert np.allclose(l, ref_l, rtol=0, atol=1e-13)


def pin_class_independence(attend):
    """A decode row equals the prefill row at the same position with the same q
    and the same pool (one mask rule for every row class); verify rows equal a
    prefill chunk over the same rows."""
    pre = wl.custom([dict(q_len=6, seq_len=45, q_start=39)], hq=4, hkv=1, d=16, dtype="bf16", seed=21)
    out_p, lse_p = attend(pre)
    for t in range(6):
        dec = pre.replace(q_len=np.array([1], np.int32), q_start=np.array([39 + t], np.int32),
                          seq_len=np.array([40 + t], np.int32), q=pre.q[t:t + 1])
        o, l = attend(dec)
        # same mask rule; equal up to BLAS summation order (shapes differ)
        assert np.allclose(o[0], out_p[t], rtol=0, atol=1e-13)
        assert np.allclose(l[0], lse_p[t], rtol=0, atol=1e-13)
    ver = pre.replace(q_len=np.array([5], np.int32), q_start=np.array([40], np.int32),
                      seq_len=np.array([45], np.int32), q=pre.q[1:6])
    o, l = attend(ver)
    assert np.allclose(o, out_p[1:6], rtol=0, atol=1e-13)
    assert np.allclose(l, lse_p[1:6], rtol=0, atol=1e-13)


def pin_gqa_replication(attend):
    """Hq = G*Hkv equals multi-head attention with each kv head copied G times
    (query head h reads kv head h // G)."""
    b = wl.custom([dict(q_len=3, seq_len=33, q_start=30), dict(q_len=1, seq_len=17)],
                  hq=6, hkv=2, d=8, dtype="f32", seed=13)
    out, lse = attend(b)
    grp = 3
    mha = b.replace(num_kv_heads=6, k_pool=np.repeat(b.k_pool, grp, axis=1),
                    v_pool=np.repeat(b.v_pool, grp, axis=1))
    o2, l2 = attend(mha)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    # and a permutation of the kv heads must change the result
    swp = b.replace(k_pool=b.k_pool[:, ::-1].copy(), v_pool=b.v_pool[:, ::-1].copy())
    o3, _ = attend(swp)
    assert not np.allclose(o3, out)


def pin_convexity(attend):
    """Softmax weights are a probability vector: min_j V_j <= O <= max_j V_j per channel."""
    b = wl.config(1)
    out, _ = attend(b)
    for row in range(b.num_rows):
        s = row
        pos = int(b.q_start[s])
        vals = np.stack([_vals(b, b.v_pool[b.block_table[s, j // 16], 0, :, j % 16])
                         for j in range(pos + 1)])
        assert np.all(out[row, 0] >= vals.min(axis=0) - 1e-15)
        assert np.all(out[row, 0] <= vals.max(axis=0) + 1e-15)


def _linearized(b, s, path):
    """One causal sequence: sequence s's context followed, at consecutive
    positions, by the K/V and queries of the tree rows ``path`` (context end
    first). Built by plain copying, in fresh pool blocks."""
    qs = int(b.q_start[s])
    n = qs + len(path)
    nb = -(-n // 16)
    src = [(int(b.block_table[s, j // 16]), j % 16) for j in range(qs)]
    src += [(int(b.block_table[s, (qs + a) // 16]), (qs + a) % 16) for a in path]
    k_tok = wl.k_token_major(b.k_pool)
    k_new = np.zeros((nb,) + k_tok.shape[1:], k_tok.dtype)
    v_new = np.zeros((nb,) + b.v_pool.shape[1:], b.v_pool.dtype)
    for j, (blk, slot) in enumerate(src):
        k_new[j // 16, :, j % 16, :] = k_tok[blk, :, slot, :]
        v_new[j // 16, :, :, j % 16] = b.v_pool[blk, :, :, slot]
    first = int(np.sum(b.q_len[:s]))
    return b.replace(q_len=np.array([len(path)], np.int32), seq_len=np.array([n], np.int32),
                     q_start=np.array([qs], np.int32), block_table=np.arange(nb, dtype=np.int32)[None],
                     num_pool_blocks=nb, q=b.q[[first + a for a in path]],
                     k_pool=wl.k_pool_layout(k_new, b.dtype), v_pool=v_new, tree_parent=None)


def _tree_batch(seed=41, dtype="bf16"):
    return wl.custom([dict(q_len=9, seq_len=50, q_start=41, tree=wl.random_tree(9, 3)),
                      dict(q_len=1, seq_len=20),
                      dict(q_len=12, seq_len=30, q_start=18, tree=wl.random_tree(12, 4, max_depth=3)),
                      dict(q_len=4, seq_len=7, q_start=3),
                      dict(q_len=5, seq_len=37, q_start=32, tree=[-1, -1, -1, -1, -1])],
                     hq=4, hkv=2, d=16, dtype=dtype, seed=seed)


def pin_tree_linearization(attend):
    """Token-tree verification: every draft row gives what ordinary causal
    attention gives for the sequence made of the context and that row's own
    path through the tree (its ancestors, then itself, at consecutive
    positions). A chain of parents is exactly the causal batch."""
    for dtype in ("bf16", "f32"):
        b = _tree_batch(dtype=dtype)
        out, lse = attend(b)
        off = b.row_offsets()
        for s in range(b.num_seqs):
            par = b.tree_parent[off[s]:off[s + 1]]
            for r in range(int(b.q_len[s])):
                path, a = [], r
                while a >= 0:
                    path.append(a)
                    a = int(par[a])
                o, l = attend(_linearized(b, s, path[::-1]))
                assert np.allclose(o[-1], out[off[s] + r], rtol=0, atol=1e-13), (dtype, s, r)
                assert np.allclose(l[-1], lse[off[s] + r], rtol=0, atol=1e-13), (dtype, s, r)
        chain = b.replace(tree_parent=np.concatenate(
            [np.arange(-1, int(q) - 1, dtype=np.int32) for q in b.q_len]))
        o1, l1 = attend(chain)
        o2, l2 = attend(b.replace(tree_parent=None))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_split_merge(mod):
    """Partial results over random disjoint key partitions (some empty), merged by
    log-sum-exp, equal the unsplit result; the merge is order independent. The
    same holds for token-tree rows, whose partitions may hide every key."""
    tb = _tree_batch(seed=43)
    t_o, t_l = mod.attend(tb)
    rng = np.random.Generator(np.random.PCG64(1))
    for _ in range(4):
        los, his = [], []
        for s in range(tb.num_seqs):
            n = int(tb.q_start[s] + tb.q_len[s])
            cut = int(rng.integers(0, n + 1))
            los.append([0, cut])
            his.append([cut, n])
        los, his = np.array(los), np.array(his)
        parts = [mod.attend_partitioned(tb, los[:, p], his[:, p]) for p in range(2)]
        mo, ml = mod.merge_partitions(np.array([p[0] for p in parts]), np.array([p[1] for p in parts]))
        assert np.allclose(mo, t_o, rtol=0, atol=1e-13) and np.allclose(ml, t_l, rtol=0, atol=1e-13)
    b = wl.custom([dict(q_len=5, seq_len=70, q_start=60), dict(q_len=1, seq_len=33),
                   dict(q_len=3, seq_len=20, q_start=3)], hq=4, hkv=2, d=16, seed=31)
    ref_o, ref_l = mod.attend(b)
    rng = np.random.Generator(np.random.PCG64(0))
    for parts in (1, 2, 3, 7):
        los, his = [], []
        for s in range(b.num_seqs):
            n = int(b.q_start[s] + b.q_len[s])
            cuts = np.sort(rng.integers(0, n + 1, size=parts - 1))
            los.append(np.concatenate([[0], cuts]))
            his.append(np.concatenate([cuts, [n]]))
        los, his = np.array(los), np.array(his)
        po, pl = [], []
        for p in range(parts):
            o, l = mod.attend_partitioned(b, los[:, p], his[:, p])
            po.append(o)
            pl.append(l)
        mo, ml = mod.merge_partitions(np.array(po), np.array(pl))
        assert np.allclose(mo, ref_o, rtol=0, atol=1e-13)
        assert np.allclose(ml, ref_l, rtol=0, atol=1e-13)
        perm = rng.permutation(parts)
        mo2, ml2 = mod.merge_partitions(np.array(po)[perm], np.array(pl)[perm])
        assert np.allclose(mo2, mo, rtol=0, atol=1e-14) and np.allclose(ml2, ml, rtol=0, atol=1e-14)
        # an extra empty partition (no keys: lse -inf) contributes nothing,
        # whatever its output slot holds
        junk_o = np.full_like(po[0], np.nan)
        junk_l = np.full_like(pl[0], -np.inf)
        mo3, ml3 = mod.merge_partitions(np.array(po + [junk_o]), np.array(pl + [junk_l]))
        assert np.array_equal(mo3, mo) and np.array_equal(ml3, ml)
    # one known two-way split checked against the closed form of the merge
    o_a, l_a = mod.attend_partitioned(b, [0, 0, 0], [16, 16, 16])
    o_b, l_b = mod.attend_partitioned(b, [16, 16, 16], [70, 33, 20])
    mo, ml = mod.merge_partitions(np.stack([o_a, o_b]), np.stack([l_a, l_b]))
    for r in range(b.num_rows):
        for h in range(4):
            la, lb = l_a[r, h], l_b[r, h]
            if np.isneginf(lb):
                assert abs(ml[r, h] - la) < 1e-13
                continue
            big = max(la, lb)
            lse = big + math.log(math.exp(la - big) + math.exp(lb - big))
            assert abs(ml[r, h] - lse) < 1e-13
            want = math.exp(la - lse) * o_a[r, h] + math.exp(lb - lse) * o_b[r, h]
            assert np.allclose(mo[r, h], want, rtol=0, atol=1e-13)
    assert np.allclose(mo, ref_o, rtol=0, atol=1e-13)


def pin_append(append_kv, gather_kv):
    """The KV append stores each new row so that gathering its position gives it
    back (the gather is pinned by the attention pins), leaves every other pool
    element unchanged, and agrees with the token-major view of the K blocks."""
    for dtype, d in (("bf16", 16), ("f32", 8), ("bf16", 24)):
        b = wl.custom([dict(q_len=5, seq_len=40, q_start=14), dict(q_len=1, seq_len=17),
                       dict(q_len=20, seq_len=36, q_start=16), dict(q_len=0, seq_len=9)],
                      hq=4, hkv=2, d=d, dtype=dtype, seed=51, extra_blocks=2)
        rng = np.random.Generator(np.random.PCG64(52))
        new_k = _store(b, rng.standard_normal((b.num_rows, 2, d)))
        new_v = _store(b, rng.standard_normal((b.num_rows, 2, d)))
        kp, vp = append_kv(b, new_k, new_v)
        changed_k = np.zeros(kp.shape, bool)
        changed_v = np.zeros(vp.shape, bool)
        k_tok = wl.k_token_major(kp)
        off = b.row_offsets()
        for s in range(b.num_seqs):
            n = int(b.q_start[s] + b.q_len[s])
            for g in range(2):
                kk, vv = gather_kv(kp, vp, b.block_table[s], g, n, dtype)
                for r in range(int(b.q_len[s])):
                    pos = int(b.q_start[s]) + r
                    row = off[s] + r
                    assert np.array_equal(kk[pos], _vals(b, new_k[row, g])), (dtype, s, r)
                    assert np.array_equal(vv[pos], _vals(b, new_v[row, g])), (dtype, s, r)
                    blk, slot = b.block_table[s, pos // 16], pos % 16
                    assert np.array_equal(k_tok[blk, g, slot], new_k[row, g])
                    changed_v[blk, g, :, slot] = True
                    x = kp.shape[-1]
                    changed_k[blk, g, :, slot, :] = True
                    assert x == wl.k_group(d, dtype)
        assert np.array_equal(kp[~changed_k], b.k_pool[~changed_k])
        assert np.array_equal(vp[~changed_v], b.v_pool[~changed_v])


ALL_PINS = [pin_single_key, pin_equal_scores, pin_two_keys, pin_golden, pin_brute_force_sdpa,
            pin_mpmath, pin_shared_equals_private, pin_class_independence, pin_gqa_replication,
            pin_convexity, pin_tree_linearization]
