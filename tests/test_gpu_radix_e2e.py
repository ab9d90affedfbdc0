"""End to end on the GPU: block tables from the radix cache, copy-on-write of
pool blocks, the KV append, then attention over the shared pool, checked
against the oracle over privately built K/V.

Each token's K/V is a fixed function of (token id, position), so equal
prefixes have equal K/V, as a model's cache would. If the cache manager, the
block copies or the append broke K/V semantics, some row would attend to a
wrong key or value and miss the oracle."""
import numpy as np
import pytest

import oracle
import prefix_shared_paged_pmattn_amd as pm
import workloads as wl
from gpu_helpers import compare, note, to_device
from prefix_shared_paged_pmattn_amd.radix import RadixCache, copy_blocks

pytestmark = pytest.mark.gpu

HQ, HKV, D, VOCAB, MAXPOS = 8, 2, 128, 40, 512


def _tables(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    tok = rng.standard_normal((2, VOCAB, HKV, D)).astype(np.float32)
    pos = rng.standard_normal((2, MAXPOS, HKV, D)).astype(np.float32) * 0.5
    return tok, pos


def _kv(tabs, tokens, positions):
    tok, pos = tabs
    t = np.asarray(tokens)
    p = np.asarray(positions)
    k = tok[0][t] + pos[0][p]
    v = tok[1][t] + pos[1][p]
    return wl.f32_to_bf16_bits(k), wl.f32_to_bf16_bits(v)   # [n][Hkv][D]


def _private_batch(seqs, q_bits, tabs):
    """The same rows over private, densely built K/V (no sharing, no cache)."""
    nb_each = [-(-len(t) // 16) for t, _ in seqs]
    total = sum(nb_each)
    k_tok = np.zeros((total, HKV, 16, D), np.uint16)
    v = np.zeros((total, HKV, D, 16), np.uint16)
    bt = np.full((len(seqs), max(nb_each)), -1, np.int32)
    base = 0
    for i, (toks, _) in enumerate(seqs):
        kk, vv = _kv(tabs, toks, range(len(toks)))
        for p in range(len(toks)):
            k_tok[base + p // 16, :, p % 16, :] = kk[p]
            v[base + p // 16, :, :, p % 16] = vv[p]
        bt[i, :nb_each[i]] = np.arange(base, base + nb_each[i])
        base += nb_each[i]
    return dict(k=wl.k_pool_layout(k_tok, "bf16"), v=v, bt=bt)


def _batch(seqs, tables, q_bits, pool_k, pool_v, num_blocks, bt_width):
    q_len = np.array([q for _, q in seqs], np.int32)
    seq_len = np.array([len(t) for t, _ in seqs], np.int32)
    bt = np.full((len(seqs), bt_width), -1, np.int32)
    for i, tb in enumerate(tables):
        bt[i, :len(tb)] = tb
    return wl.Batch(name="radix-e2e", q_len=q_len, seq_len=seq_len, q_start=seq_len - q_len,
                    block_table=bt, num_pool_blocks=num_blocks, num_q_heads=HQ, num_kv_heads=HKV,
                    head_dim=D, dtype="bf16", scale=float(np.float32(D ** -0.5)), num_kv_splits=0,
                    q=q_bits, k_pool=pool_k, v_pool=pool_v)


def _step(cache, dev, live, reqs, tabs, rng, num_blocks):
    """Admit `reqs` (token lists) and extend every live sequence by one token,
    then copy, append and attend; check against the oracle."""
    import torch
    seqs, tables, copies = [], [], []
    reused = 0
    for sid in list(live):
        toks = live[sid] + [int(rng.integers(0, VOCAB))]
        tables.append(cache.extend(sid, toks[-1:], len(toks)))
        live[sid] = toks
        seqs.append((toks, 1))
    for toks in reqs:
        sid, cl, table, cp = cache.admit(toks)
        if cl == len(toks):                      # fully cached: recompute nothing new here
            cache.release(sid)
            continue
        if cp is not None:
            copies.append(cp)
        reused += cl > 0
        live[sid] = list(toks)
        tables.append(table)
        seqs.append((list(toks), len(toks) - cl))
    copy_blocks(copies, dev["k"], dev["v"], HKV, D)
    rows_tok, rows_pos = [], []
    for toks, q in seqs:
        rows_tok += toks[len(toks) - q:]
        rows_pos += list(range(len(toks) - q, len(toks)))
    kn, vn = _kv(tabs, rows_tok, rows_pos)
    r = len(rows_tok)
    qrng = np.random.Generator(np.random.PCG64(1000 + r))
    q_bits = wl.f32_to_bf16_bits(qrng.standard_normal((r, HQ, D)).astype(np.float32))
    width = max(len(t) for t in tables)
    b = _batch(seqs, tables, q_bits, None, None, num_blocks, width)
    p = pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, num_pool_blocks=num_blocks, num_q_heads=HQ,
                num_kv_heads=HKV, head_dim=D, dtype="bf16", scale=b.scale)
    bt_dev = torch.from_numpy(b.block_table).cuda()
    to_bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    pm.kv_append(p, to_bf(kn), to_bf(vn), bt_dev, dev["k"], dev["v"])
    out = torch.empty((r, HQ, D), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((r, HQ), dtype=torch.float32, device="cuda:0")
    pm.forward(p, to_bf(q_bits), dev["k"], dev["v"], bt_dev, out, lse)
    torch.cuda.synchronize()
    priv = _private_batch(seqs, q_bits, tabs)
    ref_b = b.replace(block_table=priv["bt"], num_pool_blocks=priv["k"].shape[0], k_pool=priv["k"],
                      v_pool=priv["v"])
    note(f"  radix step: {len(seqs)} sequences, {r} rows, {len(copies)} block copies, stats {cache.stats()}")
    compare(ref_b, out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    return len(copies), reused


def test_radix_cache_end_to_end():
    import torch
    rng = np.random.Generator(np.random.PCG64(5))
    tabs = _tables(6)
    num_blocks = 36
    cache = RadixCache(num_blocks)
    dev = dict(k=torch.randn(num_blocks * HKV * 16 * D, device="cuda:0").to(torch.bfloat16),
               v=torch.randn(num_blocks * HKV * 16 * D, device="cuda:0").to(torch.bfloat16))
    docs = [rng.integers(0, VOCAB, size=int(rng.integers(20, 140))).tolist() for _ in range(4)]
    live = {}
    copies_seen = reused_seen = 0
    for step in range(12):
        reqs = []
        for _ in range(int(rng.integers(1, 4))):
            d = docs[int(rng.integers(0, len(docs)))]
            cut = int(rng.integers(1, len(d) + 1))
            reqs.append(d[:cut] + rng.integers(0, VOCAB, size=int(rng.integers(1, 20))).tolist())
        try:
            nc, nr = _step(cache, dev, live, reqs, tabs, rng, num_blocks)
            copies_seen += nc
            reused_seen += nr
        except pm.PmattnError as e:
            assert e.status == pm._lib.E_CAPACITY
            break
        # publish everything written so far; drop some sequences
        for sid in list(live):
            cache.publish(sid)
        for sid in list(live):
            if rng.random() < 0.4:
                cache.release(sid)
                del live[sid]
    st = cache.stats()
    # the run shared cached prefixes, copied partly matched blocks and evicted
    assert st["tree_nodes"] > 0 and copies_seen > 0 and reused_seen > 0 and st["evicted_nodes"] > 0, \
        (copies_seen, reused_seen, st)
