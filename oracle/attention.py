"""Exact attention over a paged, prefix-shared KV pool, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Plain and slow on
purpose: gather every key through the block table, build the causal mask as
an explicit boolean array, softmax, weighted sum. No tiling, no fusion, no
online rescaling.

What is computed, and where the pages fix it
--------------------------------------------
* The pattern is matmul -> softmax -> matmul, with QK of shape
  [tokenNum x headSize] . [headSize x kvLen] and SV of shape
  [tokenNum x kvLen] . [kvLen x headSize] (XY-Serve review page, "What carries
  the argument"; Figure 3, the dimensions table).
* Prefill-chunk, decode and verify rows are one computation that differs
  only in each row's mask (XY-Serve review, "Editorial extensions": one
  meta-kernel with row-wise mask control, no separate code paths). A query
  row at absolute position ``pos`` sees keys ``0..pos`` of its own sequence;
  the query tokens' own K/V are already in the pool (the reading taken where
  the pages are silent: the PagedAttention / prefix-caching convention they
  build on, so ``q_start + q_len <= seq_len``). Linear speculative drafts are
  causal among themselves, i.e. the same rule (Figure 8 caption).
* Entries that are masked or padded must not affect the output (XY-Serve
  review, "Assumptions & free parameters", the virtual-padding item). The page
  says they are "set to zero before softmax"; a zero *score* would still get
  weight exp(0 - max) > 0, so the only reading consistent with "do not affect
  the output" is probability exactly zero. Here: score -inf, weight exactly 0,
  and the value row is never multiplied in.
* Online softmax with rescaling equals standard softmax (same section, first
  "standard math" item), so exact softmax is the definition to compare with.
* Tree-based speculative verification (XY-Serve review, Figure 8 caption and
  the "Significance" paragraph; Medusa and SpecInfer, cited there by title):
  the draft tokens of a sequence form a tree, stored as its query rows in
  topological order with their K/V at positions q_start + r. The reading
  taken: row r sees every key below q_start (the context) and the draft keys
  of the rows on its own path to the context (its ancestors and itself),
  nothing else. A chain of parents is the linear (causal) case.
* Keys reached through shared physical blocks are the same keys as privately
  copied ones (same section: block-table management with radix-tree reuse and
  copy-on-write keeps K/V semantics).
* Split-KV with a log-sum-exp merge (reference list of the XY-Serve review:
  "Flash-Decoding for long-context inference") is exact as well; the oracle
  states each partition's (output, lse) and the merge formula directly.

Layouts (shared with the library ABI): q ``[R][Hq][d]``; k_pool
``[blocks][Hkv][d/x][16][x]`` with x = gcd(d, 16 bytes / element size), i.e.
channel ``c`` of slot ``o`` sits at ``[.., c // x, o, c % x]`` (the grouped K
layout of the PagedAttention paper's kernel, which the pages build on);
v_pool ``[blocks][Hkv][d][16]``; block_table int32 ``[B][stride]``. Query head ``h`` reads kv head ``h // (Hq // Hkv)``
(contiguous GQA groups). ``lse`` is the natural-log log-sum-exp of the scaled
scores; an empty key set gives ``lse = -inf`` and output 0.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

BLOCK = 16


def decode_values(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly. bf16 arrives as uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def gather_kv(k_pool: np.ndarray, v_pool: np.ndarray, bt_row: np.ndarray, kv_head: int,
              n_keys: int, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Logical keys 0..n_keys-1 of one sequence for one kv head, as float64 [n][d].

    Logical key j lives in physical block ``bt_row[j // 16]`` at slot ``j % 16``.
    K slots are stored as channel groups (``[blocks][Hkv][d/x][16][x]``).
    """
    j = np.arange(n_keys)
    blk = np.asarray(bt_row)[j // BLOCK]
    off = j % BLOCK
    k = k_pool[blk, kv_head, :, off, :]       # [n][d/x][x] (fancy indices lead)
    k = k.reshape(n_keys, -1)                 # [n][d]
    v = v_pool[blk, kv_head, :, off]          # [n][d] (fancy indices lead)
    return decode_values(k, dtype), decode_values(v, dtype)


def _tree_visibility(b, s: int, local_rows: np.ndarray, n_keys: int) -> np.ndarray:
    """bool [rows][n_keys]: keys a draft row may see under sequence s's token tree.

    Context keys (below q_start) are visible to every row; a draft key
    q_start + a is visible to row r iff a lies on the path from r to the
    context (walking parent links, r itself included).
    """
    off = int(np.sum(np.asarray(b.q_len)[:s]))
    ql, qs = int(b.q_len[s]), int(b.q_start[s])
    parent = np.asarray(b.tree_parent)[off:off + ql]
    vis = np.zeros((local_rows.shape[0], n_keys), dtype=bool)
    vis[:, :min(qs, n_keys)] = True
    for i, r in enumerate(local_rows):
        a = int(r)
        while a >= 0:
            if qs + a < n_keys:
                vis[i, qs + a] = True
            a = int(parent[a])
    return vis


def _attend_impl(b, rows: Optional[Sequence[int]], key_lo: Optional[np.ndarray],
                 key_hi: Optional[np.ndarray]):
    hq, hkv, d = b.num_q_heads, b.num_kv_heads, b.head_dim
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    grp = hq // hkv
    q_len = np.asarray(b.q_len, dtype=np.int64)
    q_start = np.asarray(b.q_start, dtype=np.int64)
    nseq = q_len.shape[0]
    row_off = np.zeros(nseq + 1, dtype=np.int64)
    np.cumsum(q_len, out=row_off[1:])
    total_rows = int(row_off[-1])
    want = np.arange(total_rows) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((want.shape[0], hq, d), dtype=np.float64)
    lse = np.full((want.shape[0], hq), -np.inf, dtype=np.float64)
    scale = float(np.float32(b.scale))
    seq_of = np.searchsorted(row_off, want, side="right") - 1
    for s in np.unique(seq_of):
        sel = np.nonzero(seq_of == s)[0]          # positions in the output
        r_glob = want[sel]
        pos = q_start[s] + (r_glob - row_off[s])  # absolute position of each row
        n_keys = int(pos.max()) + 1
        if n_keys > b.seq_len[s]:
            raise ValueError("a query position lies beyond seq_len")
        j = np.arange(n_keys)
        visible = j[None, :] <= pos[:, None]      # explicit causal mask [rows][keys]
        if getattr(b, "tree_parent", None) is not None:
            visible &= _tree_visibility(b, s, r_glob - row_off[s], n_keys)
        if key_lo is not None:
            visible &= (j[None, :] >= key_lo[s]) & (j[None, :] < key_hi[s])
        qf = decode_values(b.q[r_glob], b.dtype)  # [nr][Hq][d]
        for g in range(hkv):
            kk, vv = gather_kv(b.k_pool, b.v_pool, b.block_table[s], g, n_keys, b.dtype)
            for hh in range(grp):
                h = g * grp + hh
                scores = scale * (qf[:, h, :] @ kk.T)           # [nr][n]
                scores = np.where(visible, scores, -np.inf)
                m = scores.max(axis=1)
                m_safe = np.where(np.isfinite(m), m, 0.0)
                w = np.where(visible, np.exp(scores - m_safe[:, None]), 0.0)
                l = w.sum(axis=1)
                has = l > 0
                o = np.zeros((sel.shape[0], d))
                o[has] = (w[has] @ vv) / l[has, None]
                out[sel, h, :] = o
                lse[sel, h] = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return out, lse


def attend(b, rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Output ``[rows][Hq][d]`` and lse ``[rows][Hq]`` (float64) for a batch.

    ``b`` carries ``q, k_pool, v_pool, block_table, q_len, seq_len, q_start,
    num_q_heads, num_kv_heads, head_dim, dtype, scale``. ``rows`` selects
    global query rows (default: all, in order).
    """
    return _attend_impl(b, rows, None, None)


def attend_partitioned(b, key_lo: Sequence[int], key_hi: Sequence[int],
                       rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention restricted to keys ``key_lo[s] <= j < key_hi[s]`` of each sequence.

    Rows with no visible key in the range give output 0 and lse -inf.
    """
    return _attend_impl(b, rows, np.asarray(key_lo, np.int64), np.asarray(key_hi, np.int64))


def merge_partitions(parts_o: np.ndarray, parts_lse: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Combine P partial results over disjoint key sets into the full result.

    ``parts_o [P][...][d]`` are each partition's normalized outputs and
    ``parts_lse [P][...]`` their log-sum-exps. With L = ln sum_p exp(lse_p):
    out = sum_p exp(lse_p - L) * out_p, lse = L. Partitions with lse -inf
    weigh 0; if every partition is empty the result is 0 with lse -inf.
    """
    po = np.asarray(parts_o, dtype=np.float64)
    pl = np.asarray(parts_lse, dtype=np.float64)
    top = pl.max(axis=0)
    top_safe = np.where(np.isfinite(top), top, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl - top_safe[None]), 0.0)
    tot = w.sum(axis=0)
    has = tot > 0
    lse = np.where(has, top_safe + np.log(np.where(has, tot, 1.0)), -np.inf)
    coef = np.where(has[None], w / np.where(has, tot, 1.0)[None], 0.0)
    # an empty partition covers no key, so its output slot is left out of the
    # sum rather than multiplied by 0 (it may hold anything, NaN included)
    out = np.where(np.isfinite(pl)[..., None], coef[..., None] * po, 0.0).sum(axis=0)
    return out, lse


def partition_bounds(kv_len: int, parts: int) -> np.ndarray:
    """Block-aligned KV partitions ``[[lo, hi), ...]`` of keys ``0..kv_len-1``.

    The pages name split-KV (Flash-Decoding, by title) but not its boundaries;
    the reading taken: ``n_blk = ceil(kv_len/16)``, ``chunk = ceil(n_blk/P)``
    blocks, partition p = ``[p*chunk*16, min((p+1)*chunk*16, kv_len))``;
    trailing partitions may be empty (lo >= hi).
    """
    n_blk = -(-kv_len // BLOCK)
    chunk = max(1, -(-n_blk // parts))
    lo = np.minimum(np.arange(parts) * chunk * BLOCK, kv_len)
    hi = np.minimum((np.arange(parts) + 1) * chunk * BLOCK, kv_len)
    return np.stack([lo, hi], axis=1).astype(np.int64)
