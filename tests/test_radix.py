"""Host radix-tree KV cache manager (include/pmattn_radix.h), checked against
what K/V semantics require, on the CPU.

The test plays the GPU: a pool of token ids [blocks][16] stands in for the
K/V pools. Admitted sequences write their uncached tokens into the slots their
block tables name (after running the copy-on-write orders), extensions write
theirs. After every operation every live sequence must read back exactly its
own tokens through its table (block-table management plus a radix tree keep
K/V semantics under copy-on-write and eviction: XY-Serve review, "Assumptions
& free parameters"), and the reference counts must agree with the free count.
"""
import numpy as np
import pytest

import prefix_shared_paged_pmattn_amd as pm
from prefix_shared_paged_pmattn_amd import _lib
from prefix_shared_paged_pmattn_amd.radix import RadixCache

B = 16


class Model:
    def __init__(self, num_blocks):
        self.pool = np.full((num_blocks, B), -1, np.int64)
        self.live = {}          # seq -> (tokens, table)

    def copy(self, cp):
        if cp is not None:
            src, dst, slots = cp
            self.pool[dst, :slots] = self.pool[src, :slots]

    def write(self, table, tokens, lo):
        for p in range(lo, len(tokens)):
            self.pool[table[p // B], p % B] = tokens[p]

    def read(self, table, n):
        return [int(self.pool[table[p // B], p % B]) for p in range(n)]

    def check(self, cache):
        for sid, (toks, table) in self.live.items():
            assert self.read(table, len(toks)) == list(toks), f"sequence {sid} lost its K/V"
            assert len(table) == -(-len(toks) // B)
        st = cache.stats()
        refs = [cache.block_refs(b) for b in range(st["num_blocks"])]
        assert sum(r == 0 for r in refs) == st["free_blocks"]
        for toks, table in self.live.values():
            assert all(refs[b] > 0 for b in table)
        assert st["live_seqs"] == len(self.live)


def test_scenario_shares_copies_and_evicts():
    c = RadixCache(8)
    s1, cl, bt1, cp = c.admit(range(40))
    assert cl == 0 and cp is None and len(bt1) == 3
    c.publish(s1)
    s2, cl, bt2, cp = c.admit(list(range(20)) + [99] * 5)
    assert cl == 20 and bt2[0] == bt1[0] and cp == (bt1[1], bt2[1], 4)     # partial block copied
    assert c.match(list(range(40))) == 40 and c.match(list(range(20)) + [5]) == 20
    c.publish(s2)
    assert c.match(list(range(20)) + [99] * 5) == 25
    c.release(s1)
    c.release(s2)
    assert c.stats()["free_blocks"] == 4
    s3, cl, bt3, cp = c.admit(range(100, 200))                             # 7 blocks: must evict
    assert cl == 0 and c.stats()["evicted_nodes"] >= 1 and len(set(bt3.tolist())) == 7
    assert c.match(range(40)) < 40


def test_whole_request_cached_at_block_end_shares_every_block():
    c = RadixCache(16)
    s1, _, bt1, _ = c.admit(range(32))
    c.publish(s1)
    s2, cl, bt2, cp = c.admit(range(32))
    assert cl == 32 and cp is None and bt2.tolist() == bt1.tolist()
    bt2b = c.extend(s2, [7], 33)                     # the next token opens a fresh block
    assert bt2b[:2].tolist() == bt1.tolist() and bt2b[2] not in bt1


def test_capacity_error_changes_nothing():
    c = RadixCache(4)
    s1, _, _, _ = c.admit(range(50))                 # 4 blocks, all in use by a live sequence
    before = c.stats()
    with pytest.raises(pm.PmattnError) as e:
        c.admit(range(1000, 1010))
    assert e.value.status == _lib.E_CAPACITY and c.stats() == before
    with pytest.raises(pm.PmattnError):
        c.extend(s1, range(20), 70)
    assert c.stats() == before
    with pytest.raises(pm.PmattnError):
        c.release(12345)


@pytest.mark.parametrize("seed", range(6))
def test_random_workload_keeps_kv_semantics(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    nblocks = int(rng.integers(24, 80))
    c = RadixCache(nblocks)
    m = Model(nblocks)
    docs = [rng.integers(0, 50, size=int(rng.integers(5, 120))).tolist() for _ in range(6)]
    published_ever = []
    seen = dict(copies=0, reused=0)
    for step in range(600):
        op = rng.random()
        if op < 0.35 or not m.live:
            d = docs[int(rng.integers(0, len(docs)))]
            cut = int(rng.integers(0, len(d) + 1))
            toks = d[:cut] + rng.integers(0, 50, size=int(rng.integers(0, 40))).tolist()
            ev_before = c.stats()["evicted_nodes"]
            expect = c.match(toks)
            try:
                sid, cl, table, cp = c.admit(toks)
            except pm.PmattnError as e:
                assert e.status == _lib.E_CAPACITY
                continue
            # without evictions the whole cached prefix is reused
            if c.stats()["evicted_nodes"] == ev_before:
                assert cl == expect
            assert cl <= expect
            seen["copies"] += cp is not None
            seen["reused"] += cl > 0
            m.copy(cp)
            m.write(table, toks, cl)
            m.live[sid] = (toks, table.tolist())
        elif op < 0.6:
            sid = list(m.live)[int(rng.integers(0, len(m.live)))]
            toks, _ = m.live[sid]
            add = rng.integers(0, 50, size=int(rng.integers(0, 20))).tolist()
            try:
                table = c.extend(sid, add, len(toks) + len(add))
            except pm.PmattnError as e:
                assert e.status == _lib.E_CAPACITY
                continue
            toks = toks + add
            m.write(table, toks, len(toks) - len(add))
            m.live[sid] = (toks, table.tolist())
        elif op < 0.8:
            sid = list(m.live)[int(rng.integers(0, len(m.live)))]
            c.publish(sid)
            toks = m.live[sid][0]
            published_ever.append(toks)
            assert c.match(toks) == len(toks)
        else:
            sid = list(m.live)[int(rng.integers(0, len(m.live)))]
            c.release(sid)
            del m.live[sid]
        m.check(c)
    for sid in list(m.live):
        c.release(sid)
        del m.live[sid]
    m.check(c)
    st = c.stats()
    # the workload reached reuse, copy-on-write and eviction
    assert seen["copies"] > 0 and seen["reused"] > 0 and st["evicted_nodes"] > 0, (seen, st)
    assert st["live_seqs"] == 0


def test_invalid_arguments():
    with pytest.raises(pm.PmattnError):
        RadixCache(0)
    c = RadixCache(2)
    lib = _lib.load()
    import ctypes
    assert lib.pmattn_radix_admit(c._h, None, 3, None, None, None, 0, None, None) == _lib.E_INVALID
    assert lib.pmattn_radix_publish(c._h, 77) == _lib.E_INVALID


def test_copy_source_stays_pinned_when_its_leaf_is_evicted():
    """A full pool: the admit that gets a copy-on-write order must evict the
    very leaf holding the copy's source. The new sequence keeps a reference on
    that block until its next extend/publish/release, so a second admit of the
    same batch can receive it neither as a fresh block nor as its copy
    destination (one copy launch would then read and write it at once)."""
    c = RadixCache(5)
    s1, _, bt1, _ = c.admit(range(40))             # 3 blocks: [0,16) [16,32) [32,40)
    c.publish(s1)
    c.release(s1)                                  # cached in the tree only; 2 blocks free
    assert c.stats()["free_blocks"] == 2
    # match 20 tokens: block 0 shared, block 1 copied (4 slots); 3 fresh blocks
    # needed beside the shared one, so the tree's leaf is evicted
    s2, cl, bt2, cp = c.admit(list(range(20)) + [99] * 44)
    assert cl == 20 and cp is not None and cp[0] == bt1[1] and cp[2] == 4
    assert c.stats()["evicted_nodes"] >= 1
    src = cp[0]
    assert src not in bt2.tolist() and c.block_refs(src) == 1   # held for the copy
    # the pool is now full: a second admit cannot take the source block
    with pytest.raises(pm.PmattnError) as e:
        c.admit([7] * 16)
    assert e.value.status == _lib.E_CAPACITY
    c.publish(s2)                                  # the copy has run by now
    assert c.block_refs(src) == 0
    s3, _, bt3, cp3 = c.admit([7] * 16)
    assert cp3 is None and bt3.tolist() == [src]


def test_copy_source_released_by_extend_and_release():
    for finish in ("extend", "release"):
        c = RadixCache(16)
        s1, _, bt1, _ = c.admit(range(40))
        c.publish(s1)
        s2, _, _, cp = c.admit(list(range(20)) + [5])
        refs_before = c.block_refs(cp[0])
        if finish == "extend":
            c.extend(s2, [6], 22)
        else:
            c.release(s2)
        assert c.block_refs(cp[0]) == refs_before - 1
