"""Independent statement of the planner's canonical tables, and the coverage rule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The XY-Serve review page ("Core claim") decomposes each stage's attention into
tile tasks recorded in a Token-Table and a Task-Table. The library's planner
is checked against this file in two ways:

* the tables with one right answer (row -> sequence, row -> position, the
  number of KV partitions per sequence and their bounds) must match
  bit-exactly; the partition count rule and the token tiling restate the
  library's documented policy, the partition bounds follow the split-KV
  reading in ``attention.partition_bounds``, except in equal-work decode
  plans (``stream_bounds``), whose cut points are the library's policy too;
* the work list itself may come in any order, so it is checked by coverage:
  every (query row, query head, visible key) triple is covered by exactly one
  task and no task covers an invisible one.
"""
from __future__ import annotations

import numpy as np

from .attention import partition_bounds

BLOCK = 16
MAX_WAVE_ROWS = 64
MAX_TASK_ROWS = 128
CLASS_ROWS = (16, 32, 64, 128)
TASKS_PER_CU = 32
WG_TASKS_PER_2CU = 3       # 1.5 workgroup tasks per CU ...
WG_TASKS_PER_2CU_TREE = 4  # ... 2 when the plan holds a token tree
MIN_QUANTUM = 48
MAX_AUTO_SPLITS = 64
STREAM_WAVES_PER_CU = 3     # equal-work plans of 16-row tasks ...
STREAM_WAVES_PER_CU_32 = 4  # ... and of 32-row tasks
STREAM_MIN_BLOCKS = 16


def stream_applies(q_len, group, dtype="bf16", num_kv_splits=0, virtual_units=0):
    """Equal-work plans: bf16, automatic splits, no cascade group, and every
    sequence with rows a single wave task of one class: all 16-row tiles
    (q_len * G <= 16) or all 32-row tiles (16 < q_len * G <= 32)."""
    q_len = np.asarray(q_len, np.int64)
    r = q_len[q_len > 0] * group
    return (dtype == "bf16" and num_kv_splits == 0 and virtual_units == 0 and r.size > 0
            and (bool((r <= CLASS_ROWS[0]).all()) or bool(((r > CLASS_ROWS[0]) & (r <= CLASS_ROWS[1])).all())))


def stream_waves_per_cu(q_len, group):
    """Waves per CU of an equal-work plan: by the class of its tasks."""
    q_len = np.asarray(q_len, np.int64)
    return STREAM_WAVES_PER_CU if int(q_len.max()) * group <= CLASS_ROWS[0] else STREAM_WAVES_PER_CU_32


def stream_bounds(lo, hi, rows, num_kv_heads, num_cus=0, waves_per_cu=STREAM_WAVES_PER_CU):
    """Partition bounds of every unit (key ranges [lo, hi), ``rows`` > 0 for
    units with work) in an equal-work plan. The units' blocks are laid end to
    end in unit order; pieces of L blocks, L = max(16, ceil(total / (CUs x
    waves_per_cu / Hkv))), cut them; a unit's partitions are its parts of the
    pieces it meets. Returns one list of (begin, end) per unit."""
    nblk = [-(-(int(h) - int(l)) // BLOCK) if r > 0 else 0 for l, h, r in zip(lo, hi, rows)]
    total = sum(nblk)
    cus = num_cus if num_cus > 0 else 256
    per_head = max(1, cus * waves_per_cu // num_kv_heads)
    L = max(STREAM_MIN_BLOCKS, -(-total // per_head))
    out, start = [], 0
    for l, h, n in zip(lo, hi, nblk):
        b = []
        if n:
            cuts = [0] + [c - start for c in range((start // L + 1) * L, start + n, L)] + [n]
            b = [(min(int(l) + x * BLOCK, int(h)), min(int(l) + y * BLOCK, int(h))) for x, y in zip(cuts, cuts[1:])]
        out.append(b)
        start += n
    return out


def row_tables(q_len, q_start):
    """row_seq[R], row_pos[R]: each query row's sequence and absolute position."""
    q_len = np.asarray(q_len, np.int64)
    row_seq = np.repeat(np.arange(q_len.shape[0]), q_len)
    first = np.concatenate([[0], np.cumsum(q_len)[:-1]])
    row_pos = np.asarray(q_start, np.int64)[row_seq] + (np.arange(row_seq.shape[0]) - first[row_seq])
    return row_seq.astype(np.int32), row_pos.astype(np.int32)


def row_tree_masks(q_len, tree_parent):
    """Per-row visibility of the 64 keys just before the row, for token trees.

    ``tree_parent`` gives each row's parent row within its sequence (-1: the
    context). Bit k of a row's mask says whether the key k positions before
    the row may be seen: set for the row itself and each ancestor (k = row -
    ancestor), and for every k beyond the row's own index, which reaches into
    the context. Sequences whose parents form a chain (the causal rule) get
    all ones. Returns None when no sequence is a tree (or tree_parent is None).
    """
    if tree_parent is None:
        return None
    parent = np.asarray(tree_parent, np.int64)
    masks = []
    any_tree = False
    first = 0
    for ql in (int(x) for x in q_len):
        par = parent[first:first + ql]
        chain = all(int(par[r]) == r - 1 for r in range(ql))
        any_tree = any_tree or not chain
        for r in range(ql):
            if chain:
                masks.append((1 << 64) - 1)
                continue
            m = 0
            for k in range(r + 1, 64):       # keys before the tree's first row
                m |= 1 << k
            a = r
            while a >= 0:                    # the row and its ancestors
                m |= 1 << (r - a)
                a = int(par[a])
            masks.append(m)
        first += ql
    if not any_tree:
        return None
    return np.array(masks, dtype=np.uint64)


def append_units(q_len, q_start):
    """KV append units: each sequence's new tokens cut at block boundaries,
    as (seq, first row, tokens, logical block, first slot), sequence order."""
    out = []
    row = 0
    for s, (ql, qs) in enumerate(zip(q_len, q_start)):
        ql, qs = int(ql), int(qs)
        t = 0
        while t < ql:
            pos = qs + t
            n = min(ql - t, BLOCK - pos % BLOCK)
            out.append((s, row + t, n, pos // BLOCK, pos % BLOCK))
            t += n
        row += ql
    return np.array(out, dtype=np.int32).reshape(-1, 5)


def build_batch(kinds, context, pending, token_budget, reserved, max_chunk):
    """Rows each request gets in one step under the token budget (XY-Serve
    review, Figure 6 caption: chunks stay within the budget, long prefills are
    cut, slots are reserved for decode and speculative tokens). The reading:
    decode (kind 1) and verify (kind 2) requests first, in order, each whole if
    it still fits the budget; then prefill requests (kind 0), in order, share
    min(budget - reserved, budget - rows used), each taking min(pending,
    max_chunk, rows left); the first one cut short ends the prefills."""
    q = [0] * len(kinds)
    used = 0
    for i, (k, pe) in enumerate(zip(kinds, pending)):
        if k != 0 and used + pe <= token_budget:
            q[i] = int(pe)
            used += int(pe)
    left = min(token_budget - reserved, token_budget - used)
    for i, (k, pe) in enumerate(zip(kinds, pending)):
        if left <= 0:
            break
        if k != 0 or pe == 0:
            continue
        want = min(int(pe), max_chunk)
        take = min(want, left)
        q[i] = take
        left -= take
        if take < want:
            break
    return np.array(q, dtype=np.int32)


def token_tiles(q_len, q_start, group):
    """Runs of query tokens one task holds: a sequence with q_len * G <= 64
    rows is one tile (rows class 16, 32 or 64); a longer one is cut into runs
    of floor(128 / G) tokens (at least 1), rows class 128. Returns
    (seq, first token, tokens, rows class, kv end of the run)."""
    tiles = []
    for s, (ql, qs) in enumerate(zip(q_len, q_start)):
        ql, qs = int(ql), int(qs)
        if ql == 0:
            continue
        if ql * group <= MAX_WAVE_ROWS:
            cls = next(c for c in CLASS_ROWS if ql * group <= c)
            tiles.append((s, 0, ql, cls, qs + ql))
            continue
        per = max(1, MAX_TASK_ROWS // group)
        for t0 in range(0, ql, per):
            nt = min(per, ql - t0)
            tiles.append((s, t0, nt, MAX_TASK_ROWS, qs + t0 + nt))
    return tiles


def num_splits(q_len, q_start, num_kv_heads, group, num_kv_splits=0, num_cus=0, dtype="bf16", tree=False):
    """KV partitions per sequence. Explicit: the requested count for every
    sequence with rows. Automatic: a task over n blocks costs n * (2 + rows/16)
    block units. Wave tasks (<= 64 rows) and workgroup tasks (128 rows) are
    balanced separately: each kind's quantum is its total cost over
    (CUs x 32) wave tasks or (CUs x 1.5) workgroup tasks (the same when
    ``tree``: some sequence is a token tree), at least 48 units; a
    sequence gets ceil(cost of its largest tile / its kind's quantum)
    partitions, at most 64 and at most its number of blocks."""
    q_len = np.asarray(q_len, np.int64)
    q_start = np.asarray(q_start, np.int64)
    out = np.zeros(q_len.shape[0], np.int32)
    if num_kv_splits > 0:
        out[q_len > 0] = num_kv_splits
        return out
    if stream_applies(q_len, group, dtype):
        bounds = stream_bounds(np.zeros_like(q_start), q_start + q_len, q_len, num_kv_heads, num_cus,
                               stream_waves_per_cu(q_len, group))
        return np.array([len(b) for b in bounds], np.int32)
    total = [0, 0]
    last = np.zeros(q_len.shape[0], np.int64)
    kind = np.zeros(q_len.shape[0], np.int64)
    for s, _, _, cls, kv_end in token_tiles(q_len, q_start, group):
        k = 1 if cls > MAX_WAVE_ROWS else 0
        c = -(-kv_end // BLOCK) * (2 + cls // 16)
        total[k] += c * num_kv_heads
        last[s] = max(last[s], c)
        kind[s] = k
    cus = num_cus if num_cus > 0 else 256
    wg = WG_TASKS_PER_2CU_TREE if tree else WG_TASKS_PER_2CU
    quantum = [max(MIN_QUANTUM, -(-total[k] // t)) for k, t in ((0, cus * TASKS_PER_CU),
                                                                (1, cus * wg // 2))]
    for s in range(q_len.shape[0]):
        if q_len[s] == 0:
            continue
        nblk = -(-int(q_start[s] + q_len[s]) // BLOCK)
        out[s] = max(1, min(-(-int(last[s]) // quantum[kind[s]]), MAX_AUTO_SPLITS, nblk))
    return out


def seq_bounds(q_len, q_start, num_kv_heads, group, splits, num_cus=0, dtype="bf16", num_kv_splits=0):
    """Every sequence's partition bounds: ``stream_bounds`` in equal-work
    decode plans, ``partition_bounds`` (equal block chunks) otherwise."""
    q_len = np.asarray(q_len, np.int64)
    q_start = np.asarray(q_start, np.int64)
    if stream_applies(q_len, group, dtype, num_kv_splits):
        return [np.array(b, np.int64).reshape(-1, 2)
                for b in stream_bounds(np.zeros_like(q_start), q_start + q_len, q_len, num_kv_heads, num_cus,
                                       stream_waves_per_cu(q_len, group))]
    return [partition_bounds(int(q_start[s] + q_len[s]), int(p)) if p else np.zeros((0, 2), np.int64)
            for s, p in enumerate(splits)]


def split_ranges(q_len, q_start, splits, bounds=None):
    """Concatenated [begin, end) of every sequence's partitions (``bounds``:
    per-sequence bounds from ``seq_bounds``; default equal chunks)."""
    lo, hi = [], []
    for s, p in enumerate(splits):
        if p == 0:
            continue
        pb = bounds[s] if bounds is not None else partition_bounds(int(q_start[s] + q_len[s]), int(p))
        lo.append(pb[:, 0])
        hi.append(pb[:, 1])
    if not lo:
        return np.zeros(0, np.int32), np.zeros(0, np.int32)
    return np.concatenate(lo).astype(np.int32), np.concatenate(hi).astype(np.int32)


def expected_tasks(q_len, q_start, num_kv_heads, group, splits, bounds=None):
    """The set of tasks (seq, kv_head, row_begin, n_tok, pos_begin, kv_begin,
    kv_end): every tile x kv head x non-empty partition, the partition clipped
    to the tile's last position."""
    first = np.concatenate([[0], np.cumsum(np.asarray(q_len, np.int64))[:-1]])
    tasks = set()
    for s, t0, nt, _, kv_end in token_tiles(q_len, q_start, group):
        pb = bounds[s] if bounds is not None else partition_bounds(int(q_start[s] + q_len[s]), int(splits[s]))
        for g in range(num_kv_heads):
            for lo, hi in pb:
                hi = min(int(hi), kv_end)
                if lo < hi:
                    tasks.add((s, g, int(first[s]) + t0, nt, int(q_start[s]) + t0, int(lo), hi))
    return tasks


def check_coverage(items, q_len, q_start, num_kv_heads):
    """Every visible (row, kv head, key) is covered by exactly one task.

    ``items``: int array [n][>=7] of (seq, kv_head, row_begin, n_tok,
    pos_begin, kv_begin, kv_end, ...). Raises AssertionError otherwise.
    """
    items = np.asarray(items, np.int64)
    row_seq, row_pos = row_tables(q_len, q_start)
    nrows = row_seq.shape[0]
    if items.shape[0] == 0:
        assert nrows == 0, "rows exist but the work list is empty"
        return
    nt = items[:, 3]
    rep = np.repeat(np.arange(items.shape[0]), nt)
    tok = np.arange(rep.shape[0]) - np.repeat(np.cumsum(nt) - nt, nt)
    row = items[rep, 2] + tok
    kvh = items[rep, 1]
    pos = items[rep, 4] + tok
    assert (row >= 0).all() and (row < nrows).all(), "task row outside the batch"
    assert (row_seq[row] == items[rep, 0]).all(), "task row belongs to another sequence"
    assert (row_pos[row] == pos).all(), "task position disagrees with the row table"
    assert (items[:, 5] % BLOCK == 0).all(), "partition start not block aligned"
    lo = items[rep, 5]
    hi = np.minimum(items[rep, 6], pos + 1)
    assert (items[:, 6] <= items[:, 4] + items[:, 3]).all(), "task reads past its last position"
    keep = lo < hi
    row, kvh, lo, hi = row[keep], kvh[keep], lo[keep], hi[keep]
    order = np.lexsort((lo, kvh, row))
    row, kvh, lo, hi = row[order], kvh[order], lo[order], hi[order]
    key = row * num_kv_heads + kvh
    want = np.arange(nrows * num_kv_heads)
    starts = np.searchsorted(key, want, side="left")
    ends = np.searchsorted(key, want, side="right")
    assert (ends > starts).all(), "a (row, kv head) pair is not covered"
    assert (lo[starts] == 0).all(), "coverage does not start at key 0"
    assert (hi[ends - 1] == row_pos[want // num_kv_heads].astype(np.int64) + 1).all(), \
        "coverage does not end at the row's position"
    same = key[1:] == key[:-1]
    assert (hi[:-1][same] == lo[1:][same]).all(), "gap or overlap between tasks of one row"


CASCADE_AUTO_MEMBERS = 8
CASCADE_AUTO_BLOCKS = 64
CASCADE_AUTO_MIN_SPARED = 0.25   # fraction of the batch's logical keys


def cascade_groups(q_len, q_start, block_table, group, mode=1):
    """Shared-prefix runs of the cascade, in planner order, and each
    sequence's first own key.

    Candidates are sequences whose rows fit one wave task (q_len * G <= 64)
    with at least one whole block before their first query row. From the root,
    the candidates are bucketed by their block id at the current block index
    (ascending ids); a bucket of two or more extends its run while every member
    still has a whole block there with the same id, becomes a group
    (lo, hi, first member, members) and is searched further from its run's end.
    All groups of one search step are recorded before descending, and the
    first bucket is searched first. A member's own keys start at the end of
    its deepest run. Mode 2 (automatic) makes a group only of runs with at
    least 8 members spanning at least 64 blocks since the nearest group above;
    a run left out is folded into the ranges of the groups below it. Mode 2
    then drops every group unless together they spare at least a quarter of
    the batch's logical keys, counting (members - 1) x run length per group
    against the sum of q_start + q_len over sequences with rows.
    """
    n = len(q_len)
    share = [int(q_start[s]) // BLOCK for s in range(n)]
    own_lo = np.zeros(n, np.int64)
    cands = [s for s in range(n) if q_len[s] > 0 and int(q_len[s]) * group <= MAX_WAVE_ROWS and share[s] >= 1]
    min_members = CASCADE_AUTO_MEMBERS if mode == 2 else 2
    min_blocks = CASCADE_AUTO_BLOCKS if mode == 2 else 1
    groups = []
    stack = [(cands, 0, 0)]
    while stack:
        mem, depth, cover = stack.pop()
        buckets = {}
        for m in mem:
            if share[m] > depth:
                buckets.setdefault(int(block_table[m][depth]), []).append(m)
        kids = []
        for blk in sorted(buckets):
            bm = buckets[blk]
            if len(bm) < 2:
                continue
            end = depth + 1
            while all(share[m] > end and block_table[m][end] == block_table[bm[0]][end] for m in bm):
                end += 1
            kid_cover = cover
            if len(bm) >= min_members and end - cover >= min_blocks:
                groups.append((cover * BLOCK, end * BLOCK, bm[0], list(bm)))
                for m in bm:
                    own_lo[m] = end * BLOCK
                kid_cover = end
            kids.append((bm, end, kid_cover))
        stack.extend(reversed(kids))
    if mode == 2 and groups:
        spared = sum((len(g[3]) - 1) * (g[1] - g[0]) for g in groups)
        logical = sum(int(q_start[s]) + int(q_len[s]) for s in range(n) if q_len[s] > 0)
        if spared < CASCADE_AUTO_MIN_SPARED * logical:
            return [], np.zeros(n, np.int64)
    return groups, own_lo


def plan_units(q_len, q_start, block_table, num_kv_heads, group, num_kv_splits=0, num_cus=0,
               cascade=False, dtype="bf16", tree=False):
    """Units of work (real sequences, then cascade groups) with their tiles and
    KV partitions, by the same rules as ``token_tiles`` / ``num_splits`` /
    ``split_ranges`` applied to each unit's own key range [lo, hi).

    Returns dict(units=[...], vrow_src=array, groups=[...]); a unit is
    dict(virt, seq, rows, row0, pos0, lo, hi, tiles=[(t0, nt, cls, kv_end)],
    splits, bounds=[[lo, hi), ...]).
    """
    groups, own_lo = (cascade_groups(q_len, q_start, block_table, group, int(cascade)) if cascade
                      else ([], np.zeros(len(q_len), np.int64)))
    first = np.concatenate([[0], np.cumsum(np.asarray(q_len, np.int64))[:-1]]).astype(np.int64)
    units = []
    for s in range(len(q_len)):
        units.append(dict(virt=False, seq=s, rows=int(q_len[s]), row0=int(first[s]), pos0=int(q_start[s]),
                          lo=int(own_lo[s]), hi=int(q_start[s]) + int(q_len[s])))
    vrow_src = []
    for lo, hi, ts, mem in groups:
        r0 = len(vrow_src)
        for m in mem:
            vrow_src.extend(range(int(first[m]), int(first[m]) + int(q_len[m])))
        units.append(dict(virt=True, seq=ts, rows=len(vrow_src) - r0, row0=r0, pos0=hi, lo=lo, hi=hi))
    tok_wg = max(1, MAX_TASK_ROWS // group)
    for u in units:
        u["tiles"] = []
        if u["rows"] == 0:
            continue
        end = (lambda t0, nt, u=u: u["hi"] if u["virt"] else u["pos0"] + t0 + nt)
        if u["rows"] * group <= MAX_WAVE_ROWS:
            cls = next(c for c in CLASS_ROWS if u["rows"] * group <= c)
            u["tiles"].append((0, u["rows"], cls, end(0, u["rows"])))
        else:
            for t0 in range(0, u["rows"], tok_wg):
                nt = min(tok_wg, u["rows"] - t0)
                u["tiles"].append((t0, nt, MAX_TASK_ROWS, end(t0, nt)))
    stream = stream_applies(q_len, group, dtype, num_kv_splits, len(groups))
    if stream:
        sb = stream_bounds([u["lo"] for u in units], [u["hi"] for u in units], [u["rows"] for u in units],
                           num_kv_heads, num_cus, stream_waves_per_cu(q_len, group))
        for u, b in zip(units, sb):
            u["splits"], u["bounds"] = len(b), b
    elif num_kv_splits > 0:
        for u in units:
            u["splits"] = num_kv_splits if u["rows"] else 0
    else:
        total = [0, 0]
        for u in units:
            u["last"], u["kind"] = 0, 0
            for _, _, cls, kv_end in u["tiles"]:
                k = 1 if cls > MAX_WAVE_ROWS else 0
                c = -(-(kv_end - u["lo"]) // BLOCK) * (2 + cls // 16)
                total[k] += c * num_kv_heads
                u["last"] = max(u["last"], c)
                u["kind"] = k
        cus = num_cus if num_cus > 0 else 256
        wg = WG_TASKS_PER_2CU_TREE if tree else WG_TASKS_PER_2CU
        quantum = [max(MIN_QUANTUM, -(-total[0] // (cus * TASKS_PER_CU))),
                   max(MIN_QUANTUM, -(-total[1] // (cus * wg // 2)))]
        for u in units:
            nblk = -(-(u["hi"] - u["lo"]) // BLOCK)
            u["splits"] = max(1, min(-(-u["last"] // quantum[u["kind"]]), MAX_AUTO_SPLITS, nblk)) if u["rows"] else 0
    for u in units:
        if stream:
            continue
        u["bounds"] = []
        if u["splits"]:
            nblk = -(-(u["hi"] - u["lo"]) // BLOCK)
            chunk = max(1, -(-nblk // u["splits"]))
            for p in range(u["splits"]):
                u["bounds"].append((min(u["lo"] + p * chunk * BLOCK, u["hi"]),
                                    min(u["lo"] + (p + 1) * chunk * BLOCK, u["hi"])))
    return dict(units=units, vrow_src=np.array(vrow_src, np.int32), groups=groups)


def check_coverage_cascade(items, class_cascade, class_begin, vrow_src, q_len, q_start, num_kv_heads):
    """Coverage for plans with cascade classes: tasks of cascade classes hold
    virtual rows (mapped to real rows by vrow_src) over keys they see whole;
    every visible (row, kv head, key) must be covered by exactly one task."""
    row_seq, row_pos = row_tables(q_len, q_start)
    nrows = row_seq.shape[0]
    iv = []   # (row, kvh, lo, hi)
    for c in range(len(class_cascade)):
        for it in items[class_begin[c]:class_begin[c + 1]]:
            seq, kvh, r0, nt, p0, lo, hi = (int(x) for x in it[:7])
            for t in range(nt):
                if class_cascade[c]:
                    row = int(vrow_src[r0 + t])
                    assert hi <= row_pos[row], "cascade task reads keys at or past a member row"
                    iv.append((row, kvh, lo, hi))
                else:
                    assert row_seq[r0 + t] == seq and row_pos[r0 + t] == p0 + t
                    h = min(hi, p0 + t + 1)
                    if lo < h:
                        iv.append((r0 + t, kvh, lo, h))
    iv.sort()
    cur = {}
    for row, kvh, lo, hi in iv:
        want = cur.get((row, kvh), 0)
        assert lo == want, f"gap or overlap at row {row} kv head {kvh}: {want} vs {lo}"
        cur[(row, kvh)] = hi
    for row in range(nrows):
        for g in range(num_kv_heads):
            assert cur.get((row, g), 0) == int(row_pos[row]) + 1, f"row {row} kv head {g} not covered"


def streaming_tasks(items, class_begin, class_cascade, block_table):
    """Which tasks may stream their KV with non-temporal loads, and so which
    classes: a task streams when no physical block it reads is also read by a
    task of another reader. A task's reader is its row tile, named by its
    first row (item column 2), real or, in a cascade class, virtual; a task
    reads the blocks that hold keys [kv_begin, kv_end) (columns 5 and 6) of
    its block-table row (column 0). Returns (per-task flags, per-class 1 =
    all stream / 0 = none / 2 = some)."""
    readers = {}
    reads = []
    for c in range(len(class_begin) - 1):
        for it in items[class_begin[c]:class_begin[c + 1]]:
            seq, _, row0, _, _, lo, hi, _ = (int(x) for x in it[:8])
            who = ("virtual", row0) if class_cascade[c] else ("real", row0)
            blocks = {int(block_table[seq][j]) for j in range(lo // BLOCK, -(-hi // BLOCK))}
            reads.append(blocks)
            for b in blocks:
                readers.setdefault(b, set()).add(who)
    tasks = np.array([int(all(len(readers[b]) == 1 for b in blocks)) for blocks in reads], np.int32)
    classes = []
    for c in range(len(class_begin) - 1):
        part = tasks[class_begin[c]:class_begin[c + 1]]
        classes.append(1 if part.all() else 0 if not part.any() else 2)
    return tasks, np.array(classes, np.int32)
