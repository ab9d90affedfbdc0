"""GPU parity of the KV append (pmattn_kv_append) against the oracle: the pools
after the append must equal the oracle's byte for byte, and attention over the
appended pools must match the oracle's attention over them."""
import zlib

import numpy as np
import pytest

import oracle
import prefix_shared_paged_pmattn_amd as pm
import workloads as wl
from gpu_helpers import compare, make_plan, note, run_gpu, to_device

pytestmark = pytest.mark.gpu

S = dict
CASES = {
    "decode-g4-d128": (dict(hq=8, hkv=2, d=128), [S(q_len=1, seq_len=n) for n in (1, 16, 17, 300)]),
    "prefill-unaligned": (dict(hq=8, hkv=2, d=128), [S(q_len=37, seq_len=42, q_start=5), S(q_len=64, seq_len=80, q_start=16),
                                                     S(q_len=3, seq_len=30, q_start=27)]),
    "mixed-d64": (dict(hq=4, hkv=4, d=64), [S(q_len=0, seq_len=9), S(q_len=100, seq_len=130, q_start=30),
                                            S(q_len=1, seq_len=77), S(q_len=5, seq_len=21)]),
    "tree": (dict(hq=8, hkv=2, d=128), [S(q_len=12, seq_len=60, q_start=48, tree=wl.random_tree(12, 3))]),
    "f32": (dict(hq=4, hkv=2, d=128, dtype="f32"), [S(q_len=20, seq_len=36, q_start=16), S(q_len=1, seq_len=5)]),
}


def _new_rows(b, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (b.num_rows, b.num_kv_heads, b.head_dim)
    k = rng.standard_normal(shape).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    if b.dtype == "bf16":
        return wl.f32_to_bf16_bits(k), wl.f32_to_bf16_bits(v)
    return k, v


def _conv(b, a):
    import torch
    if b.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def _back(b, t):
    a = t.cpu()
    if b.dtype == "bf16":
        return a.view(__import__("torch").int16).numpy().view(np.uint16)
    return a.numpy()


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_bit_exact_then_attend(name):
    import torch
    shape, specs = CASES[name]
    b = wl.custom(specs, seed=zlib.crc32(name.encode()) % 1000, extra_blocks=2, name=name, **shape)
    note(f"append case {name}: rows={b.num_rows}")
    kn, vn = _new_rows(b, 7)
    want_k, want_v = oracle.append_kv(b, kn, vn)
    dev = to_device(b)
    p = make_plan(b)
    pm.kv_append(p, _conv(b, kn).cuda(), _conv(b, vn).cuda(), dev["bt"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    assert np.array_equal(_back(b, dev["k"]), want_k)
    assert np.array_equal(_back(b, dev["v"]), want_v)
    # attention over the appended pools, on the same device buffers
    b2 = b.replace(k_pool=want_k, v_pool=want_v)
    out, lse = run_gpu(b2, dev)
    compare(b2, out, lse)


def test_append_twice_is_idempotent_and_untouched_slots_stay():
    import torch
    b = wl.custom([S(q_len=19, seq_len=40, q_start=21), S(q_len=1, seq_len=64)], hq=8, hkv=2, d=128, seed=3,
                  extra_blocks=3)
    kn, vn = _new_rows(b, 9)
    dev = to_device(b)
    p = make_plan(b)
    ws = None
    for _ in range(2):
        ws = pm.kv_append(p, _conv(b, kn).cuda(), _conv(b, vn).cuda(), dev["bt"], dev["k"], dev["v"], workspace=ws)
    torch.cuda.synchronize()
    want_k, want_v = oracle.append_kv(b, kn, vn)
    assert np.array_equal(_back(b, dev["k"]), want_k) and np.array_equal(_back(b, dev["v"]), want_v)


def test_append_refuses_shared_slots_on_device():
    b = wl.custom([S(q_len=1, seq_len=11, q_start=10, nodes=["a"]), S(q_len=1, seq_len=30, nodes=["a"])],
                  node_blocks={"a": 1}, hq=4, hkv=2, d=64, seed=1)
    kn, vn = _new_rows(b, 1)
    dev = to_device(b)
    with pytest.raises(pm.PmattnError):
        pm.kv_append(make_plan(b), _conv(b, kn).cuda(), _conv(b, vn).cuda(), dev["bt"], dev["k"], dev["v"])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_copy_blocks_bit_exact(dtype, d):
    import torch
    from prefix_shared_paged_pmattn_amd.radix import copy_blocks
    b = wl.custom([S(q_len=1, seq_len=16 * 9)], hq=4, hkv=2, d=d, dtype=dtype, seed=4)
    dev = to_device(b)
    copies = [(0, 5, 7), (3, 1, 16), (8, 2, 1), (6, 7, 13)]
    copy_blocks(copies, dev["k"], dev["v"], b.num_kv_heads, d, dtype)
    torch.cuda.synchronize()
    kt = wl.k_token_major(b.k_pool)
    want_k, want_v = kt.copy(), b.v_pool.copy()
    for src, dst, slots in copies:
        want_k[dst, :, :slots, :] = kt[src, :, :slots, :]
        want_v[dst, :, :, :slots] = b.v_pool[src, :, :, :slots]
    assert np.array_equal(_back(b, dev["k"]), wl.k_pool_layout(want_k, dtype))
    assert np.array_equal(_back(b, dev["v"]), want_v)
