"""Helpers for GPU parity tests: move a seeded batch to the device, run the
library through its C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle
import prefix_shared_paged_pmattn_amd as pm

# Parity bars. bf16 inputs: max-abs 2e-2 and mean-abs 2e-3 over every output
# element. fp32 inputs: max-abs 1e-5. lse (natural log of scaled scores, fp32
# arithmetic on exactly-represented inputs): 1e-3 bf16, 1e-5 fp32.
TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3),
       "f32": dict(max_abs=1e-5, mean_abs=1e-6, lse=1e-5)}


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(b):
    import torch
    dev = torch.device("cuda:0")
    if b.dtype == "bf16":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)  # noqa: E731
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))  # noqa: E731
    return dict(q=conv(b.q).to(dev), k=conv(b.k_pool).to(dev), v=conv(b.v_pool).to(dev),
                bt=torch.from_numpy(np.ascontiguousarray(b.block_table, np.int32)).to(dev))


def make_plan(b, **kw):
    return pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, num_pool_blocks=b.num_pool_blocks,
                   num_q_heads=b.num_q_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                   dtype=b.dtype, scale=b.scale,
                   num_kv_splits=kw.pop("num_kv_splits", b.num_kv_splits),
                   tree_parent=kw.pop("tree_parent", b.tree_parent), **kw)


def run_gpu(b, dev=None, out_fill=float("nan"), **plan_kw):
    """Plan + forward; returns (out float64 [R][Hq][d], lse float64 [R][Hq])."""
    import torch
    dev = dev or to_device(b)
    p = make_plan(b, **plan_kw)
    et = torch.bfloat16 if b.dtype == "bf16" else torch.float32
    r, hq, d = b.num_rows, b.num_q_heads, b.head_dim
    out = torch.full((r, hq, d), out_fill, dtype=et, device="cuda:0")
    lse = torch.full((r, hq), out_fill, dtype=torch.float32, device="cuda:0")
    pm.forward(p, dev["q"], dev["k"], dev["v"], dev["bt"], out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(b, out, lse, rows=None, ref=None):
    """Check the GPU result against the oracle on all rows (or ``rows``)."""
    ro, rl = ref if ref is not None else oracle.attend(b, rows=rows)
    go = out if rows is None else out[rows]
    gl = lse if rows is None else lse[rows]
    tol = TOL[b.dtype]
    assert np.isfinite(go).all(), "non-finite output"
    err = np.abs(go - ro)
    lerr = np.abs(gl - rl)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max=float(lerr.max()))
    note(f"  parity {b.name}: {stats}")
    assert stats["max_abs"] <= tol["max_abs"], stats
    assert stats["mean_abs"] <= tol["mean_abs"], stats
    assert stats["lse_max"] <= tol["lse"], stats
    return stats


_FULL_REF = {}


def oracle_all_rows(b, key=None, workers=None):
    """``oracle.attend`` over every row of ``b``, one sequence per task on a
    thread pool (numpy and BLAS release the GIL; BLAS runs one thread per
    worker). Same function, same arithmetic per row as a single call; the
    result is cached under ``key`` for tests that compare several GPU runs of
    one workload."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    if key is not None and key in _FULL_REF:
        return _FULL_REF[key]
    off = b.row_offsets()
    seqs = [s for s in range(len(b.q_len)) if b.q_len[s] > 0]
    out = np.empty((b.num_rows, b.num_q_heads, b.head_dim), np.float64)
    lse = np.empty((b.num_rows, b.num_q_heads), np.float64)

    def one(s):
        rows = np.arange(int(off[s]), int(off[s + 1]))
        o, l = oracle.attend(b, rows=rows)
        out[rows] = o
        lse[rows] = l

    workers = workers or max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, seqs))
    if key is not None:
        _FULL_REF[key] = (out, lse)
    return out, lse
