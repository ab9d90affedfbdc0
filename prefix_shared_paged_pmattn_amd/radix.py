"""Binding of the host radix-tree KV cache manager (``include/pmattn_radix.h``)
and of the device copy-on-write of pool blocks. Argument marshalling only."""
from __future__ import annotations

import ctypes
from typing import List, Optional, Tuple

import numpy as np

from . import _lib as L
from . import _check, _dtype_code, _need_dev, _torch

BLOCK = 16


def _tok(tokens) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(tokens), dtype=np.int32)


class RadixCache:
    """``pmattn_radix_*`` over a pool of ``num_blocks`` 16-token blocks."""

    def __init__(self, num_blocks: int):
        h = ctypes.c_void_p()
        _check(L.load().pmattn_radix_create(int(num_blocks), ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            L.load().pmattn_radix_destroy(h)
            self._h = None

    def admit(self, tokens) -> Tuple[int, int, np.ndarray, Optional[Tuple[int, int, int]]]:
        """Returns (seq_id, cached_len, block_table, copy or None); copy is
        (src, dst, slots): copy slots [0, slots) of src into dst before writing."""
        t = _tok(tokens)
        n = int(t.shape[0])
        nb = -(-n // BLOCK)
        bt = np.zeros(max(nb, 1), np.int32)
        sid, cl, nc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        cp = L.BlockCopy()
        _check(L.load().pmattn_radix_admit(self._h, t.ctypes.data_as(L._i32p), n, ctypes.byref(sid),
                                           ctypes.byref(cl), bt.ctypes.data_as(L._i32p), int(bt.shape[0]),
                                           ctypes.byref(cp), ctypes.byref(nc)))
        copy = (int(cp.src), int(cp.dst), int(cp.slots)) if nc.value else None
        return int(sid.value), int(cl.value), bt[:nb].copy(), copy

    def extend(self, seq_id: int, tokens, total_tokens: int) -> np.ndarray:
        """Append tokens; returns the whole block table (``total_tokens`` = the
        sequence's length afterwards)."""
        t = _tok(tokens)
        nb = -(-int(total_tokens) // BLOCK)
        bt = np.zeros(max(nb, 1), np.int32)
        _check(L.load().pmattn_radix_extend(self._h, int(seq_id), t.ctypes.data_as(L._i32p),
                                            int(t.shape[0]), bt.ctypes.data_as(L._i32p), int(bt.shape[0])))
        return bt[:nb].copy()

    def publish(self, seq_id: int):
        _check(L.load().pmattn_radix_publish(self._h, int(seq_id)))

    def release(self, seq_id: int):
        _check(L.load().pmattn_radix_release(self._h, int(seq_id)))

    def match(self, tokens) -> int:
        t = _tok(tokens)
        m = ctypes.c_int32()
        _check(L.load().pmattn_radix_match(self._h, t.ctypes.data_as(L._i32p), int(t.shape[0]), ctypes.byref(m)))
        return int(m.value)

    def stats(self) -> dict:
        st = L.RadixStats()
        _check(L.load().pmattn_radix_stats_get(self._h, ctypes.byref(st)))
        return {k: int(getattr(st, k)) for k, _ in L.RadixStats._fields_}

    def block_refs(self, block: int) -> int:
        r = ctypes.c_int32()
        _check(L.load().pmattn_radix_block_refs(self._h, int(block), ctypes.byref(r)))
        return int(r.value)


def copy_blocks(copies: List[Tuple[int, int, int]], k_pool, v_pool, num_kv_heads: int, head_dim: int,
                dtype="bf16", stream=None):
    """``pmattn_copy_blocks``: run copy-on-write orders (src, dst, slots) on the GPU.

    Every order is checked on the host first: src and dst name blocks of the
    pools (whose element type must be ``dtype``), slots lies in 0..16, src !=
    dst and no dst repeats, so a bad order raises instead of writing outside
    the pools. The order array is copied to the device on ``stream``, the
    stream the kernel reads it on."""
    torch = _torch()
    _need_dev(k_pool, "k_pool")
    _need_dev(v_pool, "v_pool")
    code = _dtype_code(dtype)
    et = torch.bfloat16 if code == L.BF16 else torch.float32
    if k_pool.dtype != et or v_pool.dtype != et:
        raise ValueError(f"k_pool and v_pool must have dtype {et}")
    if int(head_dim) not in (64, 128) or int(num_kv_heads) < 1:
        raise ValueError("head_dim must be 64 or 128 and num_kv_heads >= 1")
    per_block = int(num_kv_heads) * BLOCK * int(head_dim)
    if k_pool.numel() != v_pool.numel() or k_pool.numel() % per_block:
        raise ValueError("k_pool and v_pool must hold the same whole number of blocks")
    nblocks = k_pool.numel() // per_block
    if not copies:
        return
    a = np.asarray(copies, np.int64).reshape(-1, 3)
    if (a[:, :2] < 0).any() or (a[:, :2] >= nblocks).any():
        raise ValueError(f"copy orders must name blocks in [0, {nblocks})")
    if (a[:, 2] < 0).any() or (a[:, 2] > BLOCK).any():
        raise ValueError("copy orders must copy 0..16 slots")
    if len(set(a[:, 1].tolist())) != a.shape[0] or (a[:, 0] == a[:, 1]).any():
        raise ValueError("copy orders need distinct destinations and src != dst")
    st = stream if stream is not None else torch.cuda.current_stream(k_pool.device)
    with torch.cuda.stream(st):
        arr = torch.tensor(a.astype(np.int32), device=k_pool.device)
    _check(L.load().pmattn_copy_blocks(ctypes.c_void_p(arr.data_ptr()), int(a.shape[0]),
                                       ctypes.c_void_p(k_pool.data_ptr()), ctypes.c_void_p(v_pool.data_ptr()),
                                       int(num_kv_heads), int(head_dim), code,
                                       ctypes.c_void_p(int(st.cuda_stream))))
    return arr
