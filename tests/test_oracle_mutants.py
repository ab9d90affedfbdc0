"""Plant plausible mistakes in a copy of the oracle (CPU only) and require that
the pin suite rejects every one of them: a dropped term, a wrong sign, index
or operand must not survive the pins."""
import importlib.util
import os
import sys
import types

import pytest

import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attention.py")

MUTANTS = {
    "diagonal-exclusive": ("visible = j[None, :] <= pos[:, None]", "visible = j[None, :] < pos[:, None]"),
    "gqa-interleaved": ("h = g * grp + hh", "h = hh * hkv + g"),
    "slot-off-by-one": ("off = j % BLOCK", "off = (j + 1) % BLOCK"),
    "block-index-wrong": ("blk = np.asarray(bt_row)[j // BLOCK]", "blk = np.asarray(bt_row)[j // (2 * BLOCK)]"),
    "v-layout-token-major": ("v = v_pool[blk, kv_head, :, off]", "v = v_pool[blk, kv_head, :, :].reshape(len(j), -1)[:, :k_pool.shape[-1]]"),
    "k-layout-token-major": ("k = k_pool[blk, kv_head, :, off, :]",
                             "k = k_pool[blk, kv_head].reshape(len(j), BLOCK, -1)[np.arange(len(j)), off]"),
    "tree-mask-dropped": ("visible &= _tree_visibility(b, s, r_glob - row_off[s], n_keys)", "pass"),
    "tree-only-self": ("            a = int(parent[a])", "            a = -1"),
    "tree-context-short": ("vis[:, :min(qs, n_keys)] = True", "vis[:, :max(0, min(qs, n_keys) - 1)] = True"),
    "scale-dropped": ("scores = scale * (qf[:, h, :] @ kk.T)", "scores = (qf[:, h, :] @ kk.T)"),
    "k-v-swapped": ("scores = scale * (qf[:, h, :] @ kk.T)", "scores = scale * (qf[:, h, :] @ vv.T)"),
    "no-normalisation": ("o[has] = (w[has] @ vv) / l[has, None]", "o[has] = (w[has] @ vv)"),
    "lse-drops-max": ("lse[sel, h] = np.where(has, m_safe + np.log(", "lse[sel, h] = np.where(has, np.log("),
    "position-from-seq-len": ("pos = q_start[s] + (r_glob - row_off[s])",
                              "pos = (np.asarray(b.seq_len)[s] - q_len[s]) + (r_glob - row_off[s])"),
    "merge-unshifted-weights": ("w = np.where(np.isfinite(pl), np.exp(pl - top_safe[None]), 0.0)",
                                "w = np.where(np.isfinite(pl), np.exp(pl), 0.0)"),
    "merge-weights-unnormalised": ("coef = np.where(has[None], w / np.where(has, tot, 1.0)[None], 0.0)",
                                   "coef = np.where(has[None], w, 0.0)"),
    "partition-lower-bound-open": ("visible &= (j[None, :] >= key_lo[s])", "visible &= (j[None, :] > key_lo[s])"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {name}"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mod = _load_mutant(name, old, new)
    failures = []
    for pin in P.ALL_PINS:
        try:
            pin(mod.attend)
        except Exception as e:          # noqa: BLE001 - any failure counts as caught
            failures.append(pin.__name__)
    try:
        P.pin_split_merge(mod)
    except Exception:                   # noqa: BLE001
        failures.append("pin_split_merge")
    assert failures, f"mutant {name} survived every pin"


def test_unmutated_copy_passes():
    src = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "<copy>", "exec"), mod.__dict__)
    for pin in P.ALL_PINS:
        pin(mod.attend)
    P.pin_split_merge(mod)


SRC_KV = os.path.join(ROOT, "oracle", "kv_cache.py")
KV_MUTANTS = {
    "append-slot-off-by-one": ("slot = pos % BLOCK", "slot = (pos + 1) % BLOCK"),
    "append-block-from-row": ("blk = int(b.block_table[s, pos // BLOCK])", "blk = int(b.block_table[s, r // BLOCK])"),
    "append-k-token-major": ("k_pool[blk, h, c // x, slot, c % x] = k_new[row, h, c]",
                             "k_pool.reshape(k_pool.shape[0], k_pool.shape[1], BLOCK, -1)[blk, h, slot, c] = k_new[row, h, c]"),
    "append-v-heads-swapped": ("v_pool[blk, h, c, slot] = v_new[row, h, c]",
                               "v_pool[blk, h, c, slot] = v_new[row, b.num_kv_heads - 1 - h, c]"),
}


@pytest.mark.parametrize("name", sorted(KV_MUTANTS))
def test_append_mutant_is_caught(name):
    import oracle
    old, new = KV_MUTANTS[name]
    src = open(SRC_KV).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {name}"
    mod = types.ModuleType(f"oracle_kv_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    with pytest.raises(Exception):     # noqa: B017 - any failure counts as caught
        P.pin_append(mod.append_kv, oracle.gather_kv)
