"""The binding uploads a plan's tables into the workspace before every pass
that reads them, unless the caller declares them resident; the library itself
never skips an upload by looking at a workspace address.

Runs on the CPU: the C library's device entry points are replaced by a
recorder (the plan itself is built by the real library, host only), and CPU
tensors stand in for device memory. Nothing is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import prefix_shared_paged_pmattn_amd as pm
from prefix_shared_paged_pmattn_amd import _lib as L
import workloads as wl


class Recorder:
    """The C ABI's device calls, recording (name, workspace address)."""

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        return getattr(self.real, name)

    def _rec(self, name, ws):
        self.calls.append((name, int(ws.value) if isinstance(ws, ctypes.c_void_p) else int(ws or 0)))
        return L.OK

    def pmattn_plan_upload(self, h, ws, n, st):
        return self._rec("upload", ws)

    def pmattn_forward(self, h, q, k, v, bt, out, lse, ws, n, st):
        return self._rec("forward", ws)

    def pmattn_forward_tasks(self, h, q, k, v, bt, out, lse, ws, n, st):
        return self._rec("tasks", ws)

    def pmattn_forward_merge(self, h, out, lse, ws, n, st):
        return self._rec("merge", ws)

    def pmattn_kv_append(self, h, kn, vn, bt, kp, vp, ws, n, st):
        return self._rec("append", ws)


@pytest.fixture
def rec(monkeypatch):
    r = Recorder(L.load())
    monkeypatch.setattr(L, "load", lambda: r)
    monkeypatch.setattr(pm, "_need_dev", lambda t, name: None)
    monkeypatch.setattr(pm, "_stream_ptr", lambda stream, like: ctypes.c_void_p(0))
    return r


def _setup():
    b = wl.custom([dict(q_len=1, seq_len=300), dict(q_len=3, seq_len=50, q_start=47)], hq=8, hkv=2, d=128,
                  seed=1, num_kv_splits=2)
    p = pm.plan(b.q_len, b.seq_len, b.q_start, b.block_table, num_pool_blocks=b.num_pool_blocks,
                num_q_heads=8, num_kv_heads=2, head_dim=128, scale=b.scale, num_kv_splits=2)
    r, d = b.num_rows, 128
    t = dict(q=torch.zeros((r, 8, d), dtype=torch.bfloat16), out=torch.zeros((r, 8, d), dtype=torch.bfloat16),
             k=torch.zeros(b.k_pool.size, dtype=torch.bfloat16), v=torch.zeros(b.v_pool.size, dtype=torch.bfloat16),
             bt=torch.from_numpy(np.ascontiguousarray(b.block_table, np.int32)),
             kn=torch.zeros((r, 2, d), dtype=torch.bfloat16), vn=torch.zeros((r, 2, d), dtype=torch.bfloat16))
    assert p.workspace_bytes > 256
    return p, t


def _ws(p):
    return torch.empty(p.workspace_bytes, dtype=torch.uint8)


def test_every_pass_uploads_first(rec):
    p, t = _setup()
    ws = _ws(p)
    pm.forward(p, t["q"], t["k"], t["v"], t["bt"], t["out"], workspace=ws)
    pm.forward(p, t["q"], t["k"], t["v"], t["bt"], t["out"], workspace=ws)   # same tensor: again
    a = ws.data_ptr()
    assert rec.calls == [("upload", a), ("forward", a), ("upload", a), ("forward", a)]


def test_new_workspace_at_a_reused_address_is_uploaded(rec):
    """A workspace freed and taken again at the same address (as a caching
    allocator hands it out) gets the tables again before the pass."""
    p, t = _setup()
    ws = _ws(p)
    pm.forward(p, t["q"], t["k"], t["v"], t["bt"], t["out"], workspace=ws)
    other = torch.empty(0, dtype=torch.uint8).set_(ws.untyped_storage())   # same memory, new tensor
    del ws
    other.fill_(0xAB)                              # another user overwrote the tables
    rec.calls.clear()
    pm.forward(p, t["q"], t["k"], t["v"], t["bt"], t["out"], workspace=other)
    assert rec.calls == [("upload", other.data_ptr()), ("forward", other.data_ptr())]


def test_fresh_workspace_uploads_and_resident_skips(rec):
    p, t = _setup()
    pm.forward(p, t["q"], t["k"], t["v"], t["bt"], t["out"])                   # allocates one
    assert [c[0] for c in rec.calls] == ["upload", "forward"]
    ws = _ws(p)
    p.upload(ws)
    rec.calls.clear()
    pm.forward(p, t["q"], t["k"], t["v"], t["bt"], t["out"], workspace=ws, resident=True)
    ws2 = pm.forward_tasks(p, t["q"], t["k"], t["v"], t["bt"], t["out"], workspace=ws, resident=True)
    pm.forward_merge(p, t["out"], None, ws2)
    assert rec.calls == [("forward", ws.data_ptr()), ("tasks", ws.data_ptr()), ("merge", ws.data_ptr())]
    with pytest.raises(ValueError):
        pm.forward(p, t["q"], t["k"], t["v"], t["bt"], t["out"], resident=True)   # no workspace given


def test_kv_append_uploads_first(rec):
    p, t = _setup()
    ws = _ws(p)
    pm.kv_append(p, t["kn"], t["vn"], t["bt"], t["k"], t["v"], workspace=ws)
    assert rec.calls == [("upload", ws.data_ptr()), ("append", ws.data_ptr())]
    rec.calls.clear()
    pm.kv_append(p, t["kn"], t["vn"], t["bt"], t["k"], t["v"], workspace=ws, resident=True)
    assert rec.calls == [("append", ws.data_ptr())]
