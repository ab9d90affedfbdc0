"""ctypes declarations of libpmattn's C ABI (include/pmattn.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpmattn.so")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_NOMEM, E_CAPACITY = range(7)
BF16, F32 = 0, 1

_i32p = ctypes.POINTER(ctypes.c_int32)


class PlanDesc(ctypes.Structure):
    # host int32 arrays, passed as addresses (const int32_t* in the C header)
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("q_len", ctypes.c_void_p),
        ("seq_len", ctypes.c_void_p),
        ("q_start", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("bt_stride", ctypes.c_int32),
        ("num_pool_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("num_kv_splits", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("work_shuffle_seed", ctypes.c_uint64),
        ("tree_parent", ctypes.c_void_p),
        ("cascade", ctypes.c_int32),
    ]


class WorkItem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("seq", "kv_head", "row_begin", "n_tok", "pos_begin", "kv_begin", "kv_end", "part")]


class MergeRow(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("rec0", "rec_stride", "nparts", "row", "q_head")]


class PlanTables(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32),
        ("row_seq", _i32p),
        ("row_pos", _i32p),
        ("num_seqs", ctypes.c_int32),
        ("num_splits", _i32p),
        ("split_offset", _i32p),
        ("split_begin", _i32p),
        ("split_end", _i32p),
        ("num_items", ctypes.c_int32),
        ("items", ctypes.POINTER(WorkItem)),
        ("num_classes", ctypes.c_int32),
        ("class_rows", _i32p),
        ("class_begin", _i32p),
        ("num_merge_rows", ctypes.c_int32),
        ("merge_rows", ctypes.POINTER(MergeRow)),
        ("num_part_records", ctypes.c_int32),
        ("row_tree_mask", ctypes.POINTER(ctypes.c_uint64)),
        ("num_append_units", ctypes.c_int32),
        ("append_units", ctypes.c_void_p),
        ("class_cascade", _i32p),
        ("num_cascade", ctypes.c_int32),
        ("cascade_lo", _i32p),
        ("cascade_hi", _i32p),
        ("cascade_seq", _i32p),
        ("cascade_row_begin", _i32p),
        ("cascade_rows", _i32p),
        ("cascade_splits", _i32p),
        ("num_virtual_rows", ctypes.c_int32),
        ("virtual_row_src", _i32p),
        ("num_rec_index", ctypes.c_int32),
        ("rec_index", _i32p),
        ("num_slots", ctypes.c_int32),
        ("slot_begin", _i32p),
        ("class_stream", _i32p),
        ("item_stream", _i32p),
        ("mixed_kernel", ctypes.c_int32),
        ("num_mix_entries", ctypes.c_int32),
        ("mix_table", _i32p),
        ("num_mix_bundles", ctypes.c_int32),
        ("mix_bundles", _i32p),
    ]


# (name, restype, argtypes) for every function the header declares.
class BlockCopy(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("src", "dst", "slots")]


class RadixStats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("tree_nodes", ctypes.c_int32), ("tree_tokens", ctypes.c_int32),
                ("live_seqs", ctypes.c_int32), ("evicted_nodes", ctypes.c_int64)]


class Request(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("kind", "context", "pending")]


class Budget(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("token_budget", "reserved", "max_chunk")]


SIGNATURES = [
    ("pmattn_plan", ctypes.c_int, [ctypes.POINTER(PlanDesc), ctypes.POINTER(ctypes.c_void_p)]),
    ("pmattn_plan_destroy", None, [ctypes.c_void_p]),
    ("pmattn_plan_workspace_bytes", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
    ("pmattn_plan_export", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(PlanTables)]),
    ("pmattn_plan_upload", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]),
    ("pmattn_forward", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]),
    ("pmattn_forward_tasks", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    ("pmattn_forward_noalloc", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]),
    ("pmattn_forward_merge", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("pmattn_merge_lse", ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    ("pmattn_kv_append", ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    ("pmattn_radix_create", ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]),
    ("pmattn_radix_destroy", None, [ctypes.c_void_p]),
    ("pmattn_radix_admit", ctypes.c_int, [ctypes.c_void_p, _i32p, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                          _i32p, ctypes.c_int32, ctypes.POINTER(BlockCopy),
                                          ctypes.POINTER(ctypes.c_int32)]),
    ("pmattn_radix_extend", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, _i32p, ctypes.c_int32,
                                           _i32p, ctypes.c_int32]),
    ("pmattn_radix_publish", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("pmattn_radix_release", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("pmattn_radix_match", ctypes.c_int, [ctypes.c_void_p, _i32p, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_int32)]),
    ("pmattn_radix_stats_get", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(RadixStats)]),
    ("pmattn_radix_block_refs", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_int32)]),
    ("pmattn_copy_blocks", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p]),
    ("pmattn_build_batch", ctypes.c_int, [ctypes.POINTER(Request), ctypes.c_int32, ctypes.POINTER(Budget),
                                          _i32p, ctypes.POINTER(ctypes.c_int32)]),
    ("pmattn_last_error", ctypes.c_char_p, []),
    ("pmattn_status_str", ctypes.c_char_p, [ctypes.c_int]),
    ("pmattn_version", ctypes.c_char_p, []),
]

_lib = None


def load() -> ctypes.CDLL:
    """Load libpmattn.so (built in-tree). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m prefix_shared_paged_pmattn_amd.build` "
                "(there is no fallback implementation)")
        # torch ships its own HIP runtime under the same soname
        # (libamdhip64.so.7) as /opt/rocm's, and the dynamic loader keeps the
        # first one loaded. Load torch's first, so that torch and this library
        # share one runtime whatever the caller touches first; the other order
        # left torch without a usable device.
        try:
            import torch  # noqa: F401
        except ImportError:  # pragma: no cover - host-only use without torch
            pass
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
