"""The KV append: this step's keys and values written into their pool slots.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Before attention runs, the new tokens' K/V are stored in the paged blocks the
block table names (XY-Serve review, "Core claim" and Figure 7, token-wise K/V
reuse over paged blocks; PagedAttention by title): query row r of sequence s
has position pos = q_start[s] + r and lives in slot pos % 16 of physical block
block_table[s][pos // 16], for every kv head. Nothing else in the pools
changes. Written out slot by slot, in the pool layouts of the library ABI:
k_pool ``[blocks][Hkv][d/x][16][x]`` (channel c of slot o at ``[c // x][o][c % x]``)
and v_pool ``[blocks][Hkv][d][16]``.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

BLOCK = 16


def append_kv(b, k_new: np.ndarray, v_new: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of ``b.k_pool`` / ``b.v_pool`` with rows ``k_new`` / ``v_new``
    (``[R][Hkv][d]``, the pools' element type) stored in their slots."""
    k_pool = b.k_pool.copy()
    v_pool = b.v_pool.copy()
    x = k_pool.shape[-1]                         # channels per 16-byte group
    row = 0
    for s in range(len(b.q_len)):
        for r in range(int(b.q_len[s])):
            pos = int(b.q_start[s]) + r
            blk = int(b.block_table[s, pos // BLOCK])
            slot = pos % BLOCK
            for h in range(b.num_kv_heads):
                for c in range(b.head_dim):
                    k_pool[blk, h, c // x, slot, c % x] = k_new[row, h, c]
                    v_pool[blk, h, c, slot] = v_new[row, h, c]
            row += 1
    return k_pool, v_pool
