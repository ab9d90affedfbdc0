"""fp64 CPU oracle for paged, prefix-shared attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg use it. It shares no code with the HIP
library (``prefix_shared_paged_pmattn_amd``) and imports nothing from it.

Contents
--------
``attention``     exact attention over a paged KV pool: gather keys through the
                  block table, explicit causal mask, softmax, output and
                  log-sum-exp, all in float64; plus attention over a key
                  partition and the log-sum-exp merge of partitions.
``kv_cache``      the KV append: this step's K/V written into their pool slots.
``plan_replica``  an independent Python statement of the planner's canonical
                  tables (row -> sequence/position, KV partitions) and the
                  coverage rule every work list must satisfy.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, brute force through library routines and an
mpmath evaluation); none is "parity unpinned".
"""
from .attention import (attend, attend_partitioned, decode_values, gather_kv, merge_partitions,
                        partition_bounds)
from .kv_cache import append_kv

__all__ = ["append_kv", "attend", "attend_partitioned", "decode_values", "gather_kv",
           "merge_partitions", "partition_bounds"]
