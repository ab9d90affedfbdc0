"""Seeded synthetic batches for paged, prefix-shared attention.

This module only *generates inputs*: batch structure (query/sequence lengths,
start positions, block tables with shared physical blocks) and random values.
It holds none of the attention arithmetic, so the fp64 oracle's tests and the
GPU library's tests/bench can both consume the same arrays without sharing
method code.

Memory layouts (the library ABI and the oracle read the same bytes):

* ``q``        ``[R][Hq][d]``       rows packed per sequence in descriptor order
* ``k_pool``   ``[num_blocks][Hkv][d/x][16][x]``   inside a block: channel
  groups of x = gcd(d, 16 bytes / element size) (8 for bf16, 4 for fp32 at
  d = 64 or 128), each holding the block's 16 tokens; see ``k_pool_layout``
* ``v_pool``   ``[num_blocks][Hkv][d][16]``   channel-major inside a block
* ``block_table`` int32 ``[B][bt_stride]``; entries past a sequence's last
  block are ``-1``.

bf16 tensors are stored as ``uint16`` bit patterns (fp32 values rounded once,
round-to-nearest-even); fp32 tensors as ``float32``.

Workload shapes follow the pages' scenarios (the XY-Serve review, "Core claim":
mixed prefill/decode/verify chunks with prefix caching; the SGLang review,
"Core claim": few-shot prompts and multi-turn chat sharing KV prefixes).
Random draws use ``numpy.random.Generator(PCG64(seed))`` in a fixed order:
structure, then physical block permutation, then q, k_pool, v_pool.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

BLOCK = 16
DTYPES = ("bf16", "f32")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    step = 1 << 22
    for a in range(0, flat_in.size, step):
        u = flat_in[a:a + step].view(np.uint32).copy()
        nan = np.isnan(flat_in[a:a + step])
        lsb = u >> 16
        lsb &= 1
        u += 0x7FFF
        u += lsb
        u >>= 16
        flat_out[a:a + step] = u
        flat_out[a:a + step][nan] = 0x7FC0
    return out


def k_group(d: int, dtype: str) -> int:
    """Channels per 16-byte group of the K pool layout: gcd(d, 16 / element size)."""
    return math.gcd(int(d), 8 if dtype == "bf16" else 4)


def k_pool_layout(k_tok: np.ndarray, dtype: str) -> np.ndarray:
    """Token-major K blocks ``[blocks][Hkv][16][d]`` -> the pool layout
    ``[blocks][Hkv][d/x][16][x]`` (a pure relayout; values are unchanged)."""
    nb, h, t, d = k_tok.shape
    x = k_group(d, dtype)
    return np.ascontiguousarray(k_tok.reshape(nb, h, t, d // x, x).transpose(0, 1, 3, 2, 4))


def k_token_major(k_pool: np.ndarray) -> np.ndarray:
    """Inverse of ``k_pool_layout``: a ``[blocks][Hkv][16][d]`` copy."""
    nb, h, g, t, x = k_pool.shape
    return np.ascontiguousarray(k_pool.transpose(0, 1, 3, 2, 4)).reshape(nb, h, t, g * x)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """i.i.d. N(0,1) drawn in float32 (in chunks, same stream as one draw), stored as ``dtype``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    step = 1 << 22
    for a in range(0, n, step):
        x = rng.standard_normal(min(step, n - a), dtype=np.float32)
        out[a:a + x.size] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out.reshape(shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Batch:
    name: str
    q_len: np.ndarray          # int32 [B]
    seq_len: np.ndarray        # int32 [B]
    q_start: np.ndarray        # int32 [B]
    block_table: np.ndarray    # int32 [B][bt_stride]
    num_pool_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # "bf16" | "f32"
    scale: float               # a float32 value (stored as Python float)
    num_kv_splits: int         # 0 = library chooses
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    # None: every row causal. Else int32 [R]: per query row, its parent row in
    # a speculative token tree (within the sequence; -1 = hangs off the
    # context). Rows are the tree's nodes in topological order.
    tree_parent: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.q_len.shape[0])

    @property
    def num_rows(self) -> int:
        return int(self.q_len.sum())

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def row_offsets(self) -> np.ndarray:
        """First global row of each sequence (rows are packed in descriptor order)."""
        off = np.zeros(self.num_seqs + 1, dtype=np.int64)
        np.cumsum(self.q_len, out=off[1:])
        return off

    def replace(self, **kw) -> "Batch":
        return dataclasses.replace(self, **kw)


# --------------------------------------------------------------------------
# structure assembly
# --------------------------------------------------------------------------

def _assemble(name: str, seqs: List[dict], node_blocks: Dict[object, int], *,
              hq: int, hkv: int, d: int, dtype: str, rng: np.random.Generator,
              num_kv_splits: int = 0, scale: Optional[float] = None,
              extra_blocks: int = 0, values: bool = True) -> Batch:
    """Build a batch from per-sequence specs.

    Each ``seqs`` entry: ``q_len, seq_len, q_start`` and ``nodes`` (a list of
    node ids whose blocks form the sequence's shared prefix, in order). The
    remaining logical blocks up to ``ceil(seq_len/16)`` are private.
    ``node_blocks`` maps node id -> number of blocks. ``extra_blocks`` adds
    pool blocks no table references. ``values=False`` skips the value draws
    (q/k_pool/v_pool are ``None``): structure-only batches for planner tests.
    """
    assert dtype in DTYPES
    used_nodes: List[object] = []
    for s in seqs:
        for n in s["nodes"]:
            if n not in used_nodes:
                used_nodes.append(n)
    n_node_blocks = sum(node_blocks[n] for n in used_nodes)
    n_private = []
    for s in seqs:
        nb = -(-s["seq_len"] // BLOCK)
        shared = sum(node_blocks[n] for n in s["nodes"])
        assert shared <= nb, (shared, nb)
        n_private.append(nb - shared)
    total = n_node_blocks + sum(n_private) + extra_blocks
    perm = rng.permutation(total).astype(np.int32)
    cursor = 0
    node_ids: Dict[object, np.ndarray] = {}
    for n in used_nodes:
        node_ids[n] = perm[cursor:cursor + node_blocks[n]]
        cursor += node_blocks[n]
    stride = max(1, max(-(-s["seq_len"] // BLOCK) for s in seqs))
    bt = np.full((len(seqs), stride), -1, dtype=np.int32)
    for i, s in enumerate(seqs):
        ids = [node_ids[n] for n in s["nodes"]]
        ids.append(perm[cursor:cursor + n_private[i]])
        cursor += n_private[i]
        row = np.concatenate(ids) if ids else np.zeros(0, np.int32)
        bt[i, :row.shape[0]] = row
    q_len = np.array([s["q_len"] for s in seqs], dtype=np.int32)
    seq_len = np.array([s["seq_len"] for s in seqs], dtype=np.int32)
    q_start = np.array([s["q_start"] for s in seqs], dtype=np.int32)
    r = int(q_len.sum())
    q = k = v = None
    if values:
        q = _normal(rng, (r, hq, d), dtype)
        k = k_pool_layout(_normal(rng, (total, hkv, BLOCK, d), dtype), dtype)
        v = _normal(rng, (total, hkv, d, BLOCK), dtype)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(d)))
    return Batch(name=name, q_len=q_len, seq_len=seq_len, q_start=q_start, block_table=bt,
                 num_pool_blocks=total, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 dtype=dtype, scale=float(np.float32(scale)), num_kv_splits=num_kv_splits,
                 q=q, k_pool=k, v_pool=v)


def custom(seqs: Sequence[dict], *, hq: int = 4, hkv: int = 2, d: int = 64, dtype: str = "bf16",
           seed: int = 0, num_kv_splits: int = 0, node_blocks: Optional[Dict[object, int]] = None,
           scale: Optional[float] = None, extra_blocks: int = 0, name: str = "custom",
           values: bool = True) -> Batch:
    """Small hand-specified batch. ``seqs`` entries need ``q_len, seq_len`` and
    optionally ``q_start`` (default ``seq_len - q_len``), ``nodes`` and
    ``tree`` (parent of each of the q_len rows; sequences without one are
    chains, i.e. causal)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    specs = []
    for s in seqs:
        specs.append(dict(q_len=int(s["q_len"]), seq_len=int(s["seq_len"]),
                          q_start=int(s.get("q_start", s["seq_len"] - s["q_len"])),
                          nodes=list(s.get("nodes", []))))
    b = _assemble(name, specs, dict(node_blocks or {}), hq=hq, hkv=hkv, d=d, dtype=dtype,
                  rng=rng, num_kv_splits=num_kv_splits, scale=scale, extra_blocks=extra_blocks,
                  values=values)
    if any("tree" in s for s in seqs):
        parents = []
        for s in seqs:
            ql = int(s["q_len"])
            tree = s.get("tree", list(range(-1, ql - 1)))
            if len(tree) != ql:
                raise ValueError("a tree needs one parent per query row")
            parents.extend(int(x) for x in tree)
        b = b.replace(tree_parent=np.array(parents, dtype=np.int32))
    return b


def random_tree(n: int, seed: int, max_depth: Optional[int] = None) -> List[int]:
    """Parents of an n-node token tree in topological order: node r hangs off a
    uniformly drawn earlier node or the context (-1), with depth <= max_depth."""
    rng = np.random.Generator(np.random.PCG64(seed))
    parents, depth = [], []
    for r in range(n):
        cands = [-1] + [a for a in range(r) if max_depth is None or depth[a] + 1 < max_depth]
        p = int(cands[int(rng.integers(0, len(cands)))])
        parents.append(p)
        depth.append(1 if p < 0 else depth[p] + 1)
    return parents


def tree_ancestors(parents: Sequence[int], r: int) -> List[int]:
    """Rows on the path from row r up to the context, r included."""
    out = []
    while r >= 0:
        out.append(r)
        r = int(parents[r])
    return out


# --------------------------------------------------------------------------
# the five workload configurations
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-f32-shared-prefix-decode",
    2: "decode-gqa-64seq-ctx512-4096",
    3: "fewshot-256x128-on-shared-2048",
    4: "mixed-prefill-decode-verify-radix",
    5: "long-decode-8x32k-paired-turns",
    6: "tree-verify-64seq-32node",
    7: "shared-prompt-decode-128seq-8k",
}


def config(idx: int, seed: Optional[int] = None, values: bool = True) -> Batch:
    """The five synthetic workloads (seed defaults to the config index).
    ``values=False`` returns the structure only (no q/K/V arrays)."""
    rng = np.random.Generator(np.random.PCG64(idx if seed is None else seed))
    name = CONFIG_NAMES[idx]
    kw = dict(values=values)
    if idx == 1:
        # 4 sequences share a 32-token prefix (2 blocks) + 16 private tokens; one decode query each.
        seqs = [dict(q_len=1, seq_len=48, q_start=47, nodes=["p"]) for _ in range(4)]
        return _assemble(name, seqs, {"p": 2}, hq=1, hkv=1, d=64, dtype="f32", rng=rng, **kw)
    if idx == 2:
        lens = rng.integers(512, 4096, size=64, endpoint=True)
        seqs = [dict(q_len=1, seq_len=int(L), q_start=int(L) - 1, nodes=[]) for L in lens]
        return _assemble(name, seqs, {}, hq=32, hkv=8, d=128, dtype="bf16", rng=rng, **kw)
    if idx == 3:
        seqs = [dict(q_len=128, seq_len=2176, q_start=2048, nodes=["prefix"]) for _ in range(256)]
        return _assemble(name, seqs, {"prefix": 128}, hq=32, hkv=8, d=128, dtype="bf16", rng=rng,
                         **kw)
    if idx == 4:
        return _config4(name, rng, values)
    if idx == 5:
        seqs = []
        for s in range(8):
            seqs.append(dict(q_len=1, seq_len=32768, q_start=32767, nodes=[("pair", s // 2)]))
        nodes = {("pair", p): 1536 for p in range(4)}
        return _assemble(name, seqs, nodes, hq=64, hkv=8, d=128, dtype="bf16", rng=rng,
                         num_kv_splits=16, **kw)
    if idx == 6:
        # Tree-based speculative verification (XY-Serve review, Figure 8 caption):
        # 64 sequences, context U{512..4096}, each verifying a 32-node draft tree
        # of depth <= 6 whose parents are drawn uniformly among earlier nodes.
        ctx = rng.integers(512, 4096, size=64, endpoint=True)
        tree_seeds = rng.integers(0, 2 ** 31, size=64)
        seqs = [dict(q_len=32, seq_len=int(c) + 32, q_start=int(c), nodes=[]) for c in ctx]
        b = _assemble(name, seqs, {}, hq=32, hkv=8, d=128, dtype="bf16", rng=rng, **kw)
        parents = [p for t in tree_seeds for p in random_tree(32, int(t), max_depth=6)]
        return b.replace(tree_parent=np.array(parents, dtype=np.int32))
    if idx == 7:
        # Many requests on one long shared prompt (the SGLang review's few-shot /
        # system-prompt sharing, at decode time): 128 sequences share an
        # 8,192-token prefix, each with a private tail U{128..1024}, one decode
        # row each; 32/8 heads, d 128.
        tail = rng.integers(128, 1024, size=128, endpoint=True)
        seqs = [dict(q_len=1, seq_len=8192 + int(t), q_start=8192 + int(t) - 1, nodes=["prompt"]) for t in tail]
        return _assemble(name, seqs, {"prompt": 512}, hq=32, hkv=8, d=128, dtype="bf16", rng=rng, **kw)
    raise KeyError(idx)


def _config4(name: str, rng: np.random.Generator, values: bool = True) -> Batch:
    """Mixed chunk: 16 prefill chunks x 512, 96 decodes, 32 verifies of 5 linear drafts.

    Prefixes come from a radix tree with branching (1, 4, 4, 4) of 256-token
    nodes (64 leaves, 1024-token root-to-leaf paths); leaf popularity is Zipf
    with s = 1.1 over ranks 1..64, ranks mapped to leaves by a seeded
    permutation. A sequence reuses the first min(1024, floor(ctx/256)*256)
    tokens of its leaf's path, where ctx is the number of tokens before its
    first query.
    """
    node_blk = 256 // BLOCK
    # structure draws
    pf_start = rng.integers(0, 4096, size=16, endpoint=True)
    dec_ctx = rng.integers(1024, 8192, size=96, endpoint=True)
    ver_ctx = rng.integers(1024, 8192, size=32, endpoint=True)
    ranks = np.arange(1, 65, dtype=np.float64)
    pz = ranks ** -1.1
    pz /= pz.sum()
    leaf_of_rank = rng.permutation(64)
    leaf = leaf_of_rank[rng.choice(64, size=16 + 96 + 32, p=pz)]

    def path(lf: int) -> List[object]:
        # node ids along the root-to-leaf path: depth k node = prefix of base-4 digits
        digits = [(lf >> 4) & 3, (lf >> 2) & 3, lf & 3]
        return [("n", 0)] + [("n", 1 + k, tuple(digits[:k + 1])) for k in range(3)]

    seqs = []
    for i in range(16):
        st = int(pf_start[i])
        seqs.append(dict(q_len=512, seq_len=st + 512, q_start=st, ctx=st))
    for i in range(96):
        c = int(dec_ctx[i])
        seqs.append(dict(q_len=1, seq_len=c, q_start=c - 1, ctx=c - 1))
    for i in range(32):
        c = int(ver_ctx[i])
        seqs.append(dict(q_len=5, seq_len=c + 5, q_start=c, ctx=c))
    nodes: Dict[object, int] = {}
    for i, s in enumerate(seqs):
        n_shared_tok = min(1024, (s.pop("ctx") // 256) * 256)
        p = path(int(leaf[i]))[: n_shared_tok // 256]
        s["nodes"] = p
        for n in p:
            nodes[n] = node_blk
    return _assemble(name, seqs, nodes, hq=32, hkv=8, d=128, dtype="bf16", rng=rng, values=values)


# --------------------------------------------------------------------------
# structure queries and batch transformations used by tests and the bench
# --------------------------------------------------------------------------

def visible_slot_mask(b: Batch) -> np.ndarray:
    """bool [num_pool_blocks][16]: slot holds a key some query row may attend."""
    vis = np.zeros((b.num_pool_blocks, BLOCK), dtype=bool)
    for s in range(b.num_seqs):
        if b.q_len[s] == 0:
            continue
        n = int(b.q_start[s] + b.q_len[s])
        j = np.arange(n)
        vis[b.block_table[s, j // BLOCK], j % BLOCK] = True
    return vis


def with_poison(b: Batch, value: float = float("nan")) -> Batch:
    """Copy of ``b`` whose pool slots that no row may see hold ``value``."""
    vis = visible_slot_mask(b)
    k = b.k_pool.copy()
    v = b.v_pool.copy()
    if b.dtype == "bf16":
        fill = f32_to_bf16_bits(np.array([value], dtype=np.float32))[0]
    else:
        fill = np.float32(value)
    blk, off = np.nonzero(~vis)
    k[blk, :, :, off, :] = fill
    v[blk, :, :, off] = fill
    return b.replace(k_pool=k, v_pool=v, name=b.name + "+poison")


def private_copy(b: Batch) -> Batch:
    """Copy of ``b`` in which no physical block is referenced by two sequences:
    every shared block is duplicated (same values) into fresh pool blocks."""
    refs: Dict[int, int] = {}
    for s in range(b.num_seqs):
        nb = -(-int(b.seq_len[s]) // BLOCK)
        for blk in b.block_table[s, :nb]:
            refs[int(blk)] = refs.get(int(blk), 0) + 1
    bt = b.block_table.copy()
    new_k = [b.k_pool]
    new_v = [b.v_pool]
    nxt = b.num_pool_blocks
    for s in range(b.num_seqs):
        nb = -(-int(b.seq_len[s]) // BLOCK)
        for j in range(nb):
            blk = int(b.block_table[s, j])
            if refs[blk] > 1:
                new_k.append(b.k_pool[blk:blk + 1])
                new_v.append(b.v_pool[blk:blk + 1])
                bt[s, j] = nxt
                nxt += 1
    return b.replace(block_table=bt, num_pool_blocks=nxt, k_pool=np.concatenate(new_k),
                     v_pool=np.concatenate(new_v), name=b.name + "+private")


def seq_kind(q_len: int) -> str:
    """Query class of a sequence by its row count: one row is a decode step,
    up to 16 rows a speculative verify, more a prefill chunk."""
    return "decode" if q_len == 1 else "verify" if q_len <= 16 else "prefill"


def subset(b: Batch, keep: np.ndarray, name: str) -> Batch:
    """Copy of ``b`` holding only the sequences where ``keep`` is true (their
    query rows, lengths and block-table rows); the pool is shared unchanged."""
    keep = np.asarray(keep, dtype=bool)
    off = b.row_offsets()
    rows = np.concatenate([np.arange(off[s], off[s + 1]) for s in np.nonzero(keep)[0]] +
                          [np.zeros(0, dtype=np.int64)])
    return b.replace(name=name, q_len=b.q_len[keep].copy(), seq_len=b.seq_len[keep].copy(),
                     q_start=b.q_start[keep].copy(), block_table=b.block_table[keep].copy(),
                     q=b.q[rows] if b.q is not None else None,
                     tree_parent=None if b.tree_parent is None else b.tree_parent[rows].copy())


def relabel(b: Batch, seed: int) -> Batch:
    """Copy of ``b`` with physical block ids permuted (pool and tables alike)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(b.num_pool_blocks).astype(np.int32)
    k = np.empty_like(b.k_pool)
    v = np.empty_like(b.v_pool)
    k[perm] = b.k_pool
    v[perm] = b.v_pool
    bt = np.where(b.block_table >= 0, perm[np.maximum(b.block_table, 0)], -1).astype(np.int32)
    return b.replace(block_table=bt, k_pool=k, v_pool=v, name=b.name + "+relabel")


def algorithmic_work(b: Batch, with_lse: bool = True) -> dict:
    """What the method must move and compute for this batch.

    Bytes: unique KV slots visible to some row (a shared block counted once)
    x 2 * Hkv * d * elem, plus Q and O (and LSE). FLOP: 4 * d * Hq per visible
    (row, key) pair. Split partials are an implementation choice and are not
    counted.
    """
    vis = visible_slot_mask(b)
    unique = int(vis.sum())
    logical = int(sum(int(b.q_start[s] + b.q_len[s]) for s in range(b.num_seqs) if b.q_len[s] > 0))
    pairs = 0
    off = b.row_offsets()
    for s in range(b.num_seqs):
        ql, qs = int(b.q_len[s]), int(b.q_start[s])
        if b.tree_parent is None:
            pairs += ql * (qs + 1) + ql * (ql - 1) // 2
        else:
            par = b.tree_parent[off[s]:off[s] + ql]
            pairs += sum(qs + len(tree_ancestors(par, r)) for r in range(ql))
    e = b.elem_bytes
    hq, hkv, d, r = b.num_q_heads, b.num_kv_heads, b.head_dim, b.num_rows
    kv_bytes = unique * 2 * hkv * d * e
    q_bytes = r * hq * d * e
    o_bytes = r * hq * d * e
    lse_bytes = r * hq * 4 if with_lse else 0
    return dict(unique_kv_tokens=unique, logical_kv_tokens=logical, visible_pairs=pairs,
                flop=4 * d * hq * pairs, kv_bytes_unique=kv_bytes,
                kv_bytes_logical=logical * 2 * hkv * d * e, q_bytes=q_bytes, o_bytes=o_bytes,
                lse_bytes=lse_bytes, bytes=kv_bytes + q_bytes + o_bytes + lse_bytes)
