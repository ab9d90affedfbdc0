"""Python binding of libpmattn: paged, prefix-shared mixed attention on gfx950.

Argument marshalling only. Every step of the computation runs in the HIP
kernels of ``libpmattn.so``; torch tensors only provide device memory and the
stream. The names mirror the C ABI (``include/pmattn.h``):

* ``plan(...)``      -> ``pmattn_plan`` (host only; returns a :class:`Plan`)
* ``forward(...)``   -> ``pmattn_forward``
* ``merge_lse(...)`` -> ``pmattn_merge_lse``

Host-side shape, dtype and device checks happen here before any launch, so a
mis-sized tensor is an exception, never an out-of-bounds kernel access.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib as L

__all__ = ["Plan", "PmattnError", "plan", "forward", "forward_tasks", "forward_merge", "forward_noalloc",
           "merge_lse", "kv_append", "build_batch", "version", "BF16", "F32"]

BF16, F32 = L.BF16, L.F32


class PmattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        lib = L.load()
        super().__init__(f"{lib.pmattn_status_str(status).decode()}: {msg}")
        self.status = status


def _check(status: int):
    if status != L.OK:
        raise PmattnError(status, L.load().pmattn_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _dtype_code(dtype) -> int:
    if dtype in ("bf16", BF16):
        return BF16
    if dtype in ("f32", "fp32", F32):
        return F32
    raise ValueError(f"unknown dtype {dtype!r}")


def version() -> str:
    return L.load().pmattn_version().decode()


class Plan:
    """Owns a ``pmattn_plan_t``. Build with :func:`plan`."""

    def __init__(self, handle: ctypes.c_void_p, shape: dict):
        self._h = handle
        self.shape = shape
        n = ctypes.c_size_t()
        _check(L.load().pmattn_plan_workspace_bytes(self._h, ctypes.byref(n)))
        self.workspace_bytes = int(n.value)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            try:
                L.load().pmattn_plan_destroy(h)
            except Exception:  # interpreter shutdown
                pass
            self._h = None

    @property
    def handle(self):
        return self._h

    def tables(self) -> dict:
        """Copies of the canonical tables (``pmattn_plan_export``)."""
        t = L.PlanTables()
        _check(L.load().pmattn_plan_export(self._h, ctypes.byref(t)))

        def arr(ptr, n):
            return np.ctypeslib.as_array(ptr, shape=(n,)).copy() if n and ptr else np.zeros(0, np.int32)

        nsp = int(np.ctypeslib.as_array(t.split_offset, shape=(t.num_seqs + 1,))[-1])
        items = np.zeros((t.num_items, 8), np.int32)
        if t.num_items:
            raw = ctypes.cast(t.items, ctypes.POINTER(ctypes.c_int32))
            items = np.ctypeslib.as_array(raw, shape=(t.num_items * 8,)).reshape(-1, 8).copy()
        merge = np.zeros((t.num_merge_rows, 5), np.int32)
        if t.num_merge_rows:
            raw = ctypes.cast(t.merge_rows, ctypes.POINTER(ctypes.c_int32))
            merge = np.ctypeslib.as_array(raw, shape=(t.num_merge_rows * 5,)).reshape(-1, 5).copy()
        return dict(
            row_seq=arr(t.row_seq, t.num_rows), row_pos=arr(t.row_pos, t.num_rows),
            num_splits=arr(t.num_splits, t.num_seqs),
            split_offset=arr(t.split_offset, t.num_seqs + 1),
            split_begin=arr(t.split_begin, nsp), split_end=arr(t.split_end, nsp),
            items=items, class_rows=arr(t.class_rows, t.num_classes),
            class_begin=arr(t.class_begin, t.num_classes + 1), merge_rows=merge,
            num_part_records=int(t.num_part_records),
            row_tree_mask=(np.ctypeslib.as_array(t.row_tree_mask, shape=(t.num_rows,)).copy()
                           if t.row_tree_mask and t.num_rows else None),
            append_units=(np.ctypeslib.as_array(ctypes.cast(t.append_units, ctypes.POINTER(ctypes.c_int32)),
                                                shape=(t.num_append_units * 5,)).reshape(-1, 5).copy()
                          if t.num_append_units else np.zeros((0, 5), np.int32)),
            class_cascade=arr(t.class_cascade, t.num_classes),
            cascade=dict(lo=arr(t.cascade_lo, t.num_cascade), hi=arr(t.cascade_hi, t.num_cascade),
                         seq=arr(t.cascade_seq, t.num_cascade),
                         row_begin=arr(t.cascade_row_begin, t.num_cascade),
                         rows=arr(t.cascade_rows, t.num_cascade),
                         splits=arr(t.cascade_splits, t.num_cascade)),
            virtual_row_src=arr(t.virtual_row_src, t.num_virtual_rows),
            rec_index=arr(t.rec_index, t.num_rec_index),
            slot_begin=arr(t.slot_begin, t.num_slots + 1) if t.num_slots else np.zeros(0, np.int32),
            class_stream=arr(t.class_stream, t.num_classes),
            item_stream=arr(t.item_stream, t.num_items),
            mixed_kernel=int(t.mixed_kernel),
            mix_table=arr(t.mix_table, t.num_mix_entries),
            mix_bundles=arr(t.mix_bundles, 4 * t.num_mix_bundles))

    def upload(self, workspace, stream=None):
        """``pmattn_plan_upload``: copy the plan's tables (work list, merge
        list, row tables) into ``workspace``, asynchronously on ``stream``."""
        _need_dev(workspace, "workspace")
        nbytes = workspace.numel() * workspace.element_size()
        _check(L.load().pmattn_plan_upload(self._h, ctypes.c_void_p(workspace.data_ptr()),
                                           nbytes, _stream_ptr(stream, workspace)))


def plan(q_len, seq_len, q_start, block_table, *, num_pool_blocks: int, num_q_heads: int,
         num_kv_heads: int, head_dim: int, dtype="bf16", scale: float, num_kv_splits: int = 0,
         num_cus: int = 0, work_shuffle_seed: int = 0, tree_parent=None, cascade: int = 2) -> Plan:
    """``pmattn_plan`` over host arrays (int32-convertible). ``tree_parent``:
    None, or one int per query row (parent row within its sequence, -1 for the
    context) for speculative token trees. ``cascade``: 0 off, 1 every shared
    prefix run of decode/verify sequences, 2 (default) automatic."""
    ql, sl, qs = _i32(q_len), _i32(seq_len), _i32(q_start)
    bt = _i32(block_table)
    if bt.ndim != 2:
        raise ValueError("block_table must be 2-D [num_seqs][bt_stride]")
    b = int(ql.shape[0])
    if sl.shape != (b,) or qs.shape != (b,) or bt.shape[0] != b:
        raise ValueError("q_len, seq_len, q_start and block_table disagree on num_seqs")
    rows = int(ql.sum())
    tp = None
    if tree_parent is not None:
        tp = _i32(tree_parent)
        if tp.shape != (rows,):
            raise ValueError("tree_parent needs one entry per query row")
    # (positional, in the field order of pmattn_plan_desc)
    d = L.PlanDesc(b, ql.ctypes.data, sl.ctypes.data, qs.ctypes.data, bt.ctypes.data, int(bt.shape[1]),
                   int(num_pool_blocks), 16, int(num_q_heads), int(num_kv_heads), int(head_dim),
                   _dtype_code(dtype), float(scale), int(num_kv_splits), int(num_cus), int(work_shuffle_seed),
                   tp.ctypes.data if tp is not None else None, int(cascade))
    h = ctypes.c_void_p()
    _check(L.load().pmattn_plan(ctypes.byref(d), ctypes.byref(h)))
    shape = dict(num_seqs=b, num_rows=rows, bt_stride=int(bt.shape[1]),
                 num_pool_blocks=int(num_pool_blocks), hq=int(num_q_heads), hkv=int(num_kv_heads),
                 d=int(head_dim), dtype=_dtype_code(dtype))
    return Plan(h, shape)


# --------------------------------------------------------------------------
# device-side calls (torch tensors supply memory and stream)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _need_dev(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a torch tensor on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(stream, like) -> ctypes.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    return ctypes.c_void_p(int(stream.cuda_stream))


def _elem_dtype(code):
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


def _forward_args(p: Plan, q, k_pool, v_pool, block_table, out, lse, workspace, stream, resident):
    torch = _torch()
    s = p.shape
    et = _elem_dtype(s["dtype"])
    r, hq, hkv, d = s["num_rows"], s["hq"], s["hkv"], s["d"]
    pool_elems = s["num_pool_blocks"] * hkv * 16 * d
    checks = [(q, "q", et, r * hq * d, True), (out, "out", et, r * hq * d, True),
              (k_pool, "k_pool", et, pool_elems, False), (v_pool, "v_pool", et, pool_elems, False),
              (block_table, "block_table", torch.int32, s["num_seqs"] * s["bt_stride"], True)]
    if lse is not None:
        checks.append((lse, "lse", torch.float32, r * hq, True))
    for t, name, dt, n, exact in checks:
        _need_dev(t, name)
        if t.dtype != dt:
            raise ValueError(f"{name} must have dtype {dt}, got {t.dtype}")
        if (t.numel() != n) if exact else (t.numel() < n):
            raise ValueError(f"{name} has {t.numel()} elements, expected {'' if exact else '>= '}{n}")
        if t.data_ptr() % 16:
            raise ValueError(f"{name} must be 16-byte aligned")
    return _workspace(p, workspace, q, stream, resident)


def _workspace(p: Plan, workspace, like, stream, resident=False):
    """The caller's workspace (checked), or a fresh one, with the plan's tables
    uploaded into it unless ``resident`` says the caller already did so
    (``p.upload(workspace)``) and nothing has written it since. The library
    never decides that by itself: memory taken from an allocator may have held
    anything, including an earlier copy of these tables at the same address."""
    torch = _torch()
    if workspace is None:
        if resident:
            raise ValueError("resident=True needs the workspace the plan was uploaded into")
        workspace = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=like.device)
    _need_dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < p.workspace_bytes:
        raise ValueError(f"workspace has {ws_bytes} bytes, plan needs {p.workspace_bytes}")
    if not resident:
        p.upload(workspace, stream)
    return workspace, ws_bytes


def _vp(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def forward(p: Plan, q, k_pool, v_pool, block_table, out, lse=None, workspace=None, stream=None,
            resident=False):
    """``pmattn_forward``. Tensors: q/out ``[R][Hq][d]``; k_pool
    ``[blocks][Hkv][d/x][16][x]`` (x = 16 bytes / element size); v_pool ``[blocks][Hkv][d][16]`` (element type of
    the plan); block_table int32 ``[B][stride]``; lse float32 ``[R][Hq]`` or
    None; workspace: a uint8 tensor of at least ``p.workspace_bytes`` (None:
    a fresh one). The plan's tables are uploaded into the workspace first,
    unless ``resident`` (the caller ran ``p.upload(workspace)`` and nothing has
    written the workspace since)."""
    workspace, ws_bytes = _forward_args(p, q, k_pool, v_pool, block_table, out, lse, workspace, stream,
                                        resident)
    _check(L.load().pmattn_forward(p.handle, _vp(q), _vp(k_pool), _vp(v_pool), _vp(block_table),
                                   _vp(out), _vp(lse), _vp(workspace), ws_bytes,
                                   _stream_ptr(stream, q)))
    return out, lse


def forward_tasks(p: Plan, q, k_pool, v_pool, block_table, out, lse=None, workspace=None,
                  stream=None, resident=False):
    """``pmattn_forward_tasks``: pass 1 of :func:`forward` (the tile tasks).
    Returns the workspace, which :func:`forward_merge` must be given."""
    workspace, ws_bytes = _forward_args(p, q, k_pool, v_pool, block_table, out, lse, workspace, stream,
                                        resident)
    _check(L.load().pmattn_forward_tasks(p.handle, _vp(q), _vp(k_pool), _vp(v_pool),
                                         _vp(block_table), _vp(out), _vp(lse), _vp(workspace),
                                         ws_bytes, _stream_ptr(stream, q)))
    return workspace


def forward_noalloc(p: Plan, q, k_pool, v_pool, block_table, out, lse=None, stream=None):
    """``pmattn_forward_noalloc``: :func:`forward` without a workspace (the
    library's static device scratch holds the tables and partials; calls on
    one GPU must not overlap). Tensors as for :func:`forward`."""
    torch = _torch()
    s = p.shape
    et = _elem_dtype(s["dtype"])
    r, hq, hkv, d = s["num_rows"], s["hq"], s["hkv"], s["d"]
    pool_elems = s["num_pool_blocks"] * hkv * 16 * d
    checks = [(q, "q", et, r * hq * d, True), (out, "out", et, r * hq * d, True),
              (k_pool, "k_pool", et, pool_elems, False), (v_pool, "v_pool", et, pool_elems, False),
              (block_table, "block_table", torch.int32, s["num_seqs"] * s["bt_stride"], True)]
    if lse is not None:
        checks.append((lse, "lse", torch.float32, r * hq, True))
    for t, name, dt, n, exact in checks:
        _need_dev(t, name)
        if t.dtype != dt:
            raise ValueError(f"{name} must have dtype {dt}, got {t.dtype}")
        if (t.numel() != n) if exact else (t.numel() < n):
            raise ValueError(f"{name} has {t.numel()} elements, expected {'' if exact else '>= '}{n}")
        if t.data_ptr() % 16:
            raise ValueError(f"{name} must be 16-byte aligned")
    _check(L.load().pmattn_forward_noalloc(p.handle, _vp(q), _vp(k_pool), _vp(v_pool), _vp(block_table),
                                           _vp(out), _vp(lse), _stream_ptr(stream, q)))
    return out, lse


PREFILL, DECODE, VERIFY = 0, 1, 2


def build_batch(kinds, context, pending, *, token_budget: int, reserved: int, max_chunk: int) -> np.ndarray:
    """``pmattn_build_batch``: query rows each request gets this step (host only)."""
    k, c, pe = _i32(kinds), _i32(context), _i32(pending)
    n = int(k.shape[0])
    if c.shape != (n,) or pe.shape != (n,):
        raise ValueError("kinds, context and pending must have one entry per request")
    reqs = (L.Request * max(n, 1))()
    for i in range(n):
        reqs[i] = L.Request(int(k[i]), int(c[i]), int(pe[i]))
    q = np.zeros(max(n, 1), np.int32)
    total = ctypes.c_int32()
    bud = L.Budget(int(token_budget), int(reserved), int(max_chunk))
    _check(L.load().pmattn_build_batch(reqs, n, ctypes.byref(bud), q.ctypes.data_as(L._i32p),
                                       ctypes.byref(total)))
    return q[:n].copy()


def kv_append(p: Plan, k_new, v_new, block_table, k_pool, v_pool, workspace=None, stream=None,
              resident=False):
    """``pmattn_kv_append``: write this step's K/V rows (``k_new``, ``v_new``
    ``[R][Hkv][d]``, the plan's element type) into their pool slots, in place.
    ``workspace`` and ``resident`` as for :func:`forward`."""
    torch = _torch()
    s = p.shape
    et = _elem_dtype(s["dtype"])
    r, hkv, d = s["num_rows"], s["hkv"], s["d"]
    pool_elems = s["num_pool_blocks"] * hkv * 16 * d
    for t, name, dt, n, exact in ((k_new, "k_new", et, r * hkv * d, True),
                                  (v_new, "v_new", et, r * hkv * d, True),
                                  (k_pool, "k_pool", et, pool_elems, False),
                                  (v_pool, "v_pool", et, pool_elems, False),
                                  (block_table, "block_table", torch.int32,
                                   s["num_seqs"] * s["bt_stride"], True)):
        _need_dev(t, name)
        if t.dtype != dt:
            raise ValueError(f"{name} must have dtype {dt}, got {t.dtype}")
        if (t.numel() != n) if exact else (t.numel() < n):
            raise ValueError(f"{name} has {t.numel()} elements, expected {'' if exact else '>= '}{n}")
        if t.data_ptr() % 16:
            raise ValueError(f"{name} must be 16-byte aligned")
    workspace, ws_bytes = _workspace(p, workspace, k_pool, stream, resident)
    _check(L.load().pmattn_kv_append(p.handle, _vp(k_new), _vp(v_new), _vp(block_table),
                                     _vp(k_pool), _vp(v_pool), _vp(workspace), ws_bytes,
                                     _stream_ptr(stream, k_pool)))
    return workspace


def forward_merge(p: Plan, out, lse, workspace, stream=None):
    """``pmattn_forward_merge``: pass 2 of :func:`forward` (merge of split
    partials). ``workspace`` must be the one pass 1 (:func:`forward_tasks`)
    ran on, which holds the plan's tables and the partial records."""
    _need_dev(out, "out")
    _need_dev(workspace, "workspace")
    if lse is not None:
        _need_dev(lse, "lse")
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < p.workspace_bytes:
        raise ValueError(f"workspace has {ws_bytes} bytes, plan needs {p.workspace_bytes}")
    _check(L.load().pmattn_forward_merge(p.handle, _vp(out), _vp(lse), _vp(workspace), ws_bytes,
                                         _stream_ptr(stream, out)))


def merge_lse(part_o, part_lse, out, lse=None, stream=None):
    """``pmattn_merge_lse``: part_o float32 ``[P][rows][H][d]``, part_lse
    float32 ``[P][rows][H]``, out ``[rows][H][d]`` (bf16 or float32), lse
    float32 ``[rows][H]`` or None."""
    torch = _torch()
    if part_o.dim() != 4:
        raise ValueError("part_o must be [P][rows][H][d]")
    P_, rows, h, d = part_o.shape
    for t, name, dt, shp in ((part_o, "part_o", torch.float32, (P_, rows, h, d)),
                             (part_lse, "part_lse", torch.float32, (P_, rows, h))):
        _need_dev(t, name)
        if t.dtype != dt or tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {dt} of shape {shp}")
    _need_dev(out, "out")
    if tuple(out.shape) != (rows, h, d) or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be bf16/float32 of shape [rows][H][d]")
    if lse is not None:
        _need_dev(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (rows, h):
            raise ValueError("lse must be float32 [rows][H]")
    code = BF16 if out.dtype == torch.bfloat16 else F32
    _check(L.load().pmattn_merge_lse(P_, rows, h, d, _vp(part_o), _vp(part_lse), _vp(out), code,
                                     _vp(lse), _stream_ptr(stream, out)))
    return out, lse
