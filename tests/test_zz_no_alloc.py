"""pmattn_forward_noalloc (the entry point for callers that cannot allocate)
against pmattn_forward, through the C ABI: two calls in a row on one GPU, the
second with a smaller batch, each bit-identical to pmattn_forward's output and
within the oracle bars; and the host-side refusal of a plan larger than the
static scratch."""
import numpy as np
import pytest

import prefix_shared_paged_pmattn_amd as pm
import workloads as wl
from gpu_helpers import compare, make_plan, note, run_gpu, to_device


def _noalloc(b, dev, **kw):
    import torch
    p = make_plan(b, **kw)
    et = torch.bfloat16 if b.dtype == "bf16" else torch.float32
    out = torch.full((b.num_rows, b.num_q_heads, b.head_dim), float("nan"), dtype=et, device="cuda:0")
    lse = torch.full((b.num_rows, b.num_q_heads), float("nan"), dtype=torch.float32, device="cuda:0")
    pm.forward_noalloc(p, dev["q"], dev["k"], dev["v"], dev["bt"], out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.gpu
def test_noalloc_matches_forward_two_calls_shrinking():
    big = wl.custom([dict(q_len=1, seq_len=n) for n in (900, 33, 4000)] +
                    [dict(q_len=5, seq_len=300, q_start=295), dict(q_len=150, seq_len=400, q_start=250)],
                    hq=8, hkv=2, d=128, seed=31, num_kv_splits=0, name="noalloc-big")
    small = wl.custom([dict(q_len=1, seq_len=70), dict(q_len=3, seq_len=20, q_start=17)],
                      hq=8, hkv=2, d=128, seed=32, num_kv_splits=2, name="noalloc-small")
    assert make_plan(big).workspace_bytes > make_plan(small).workspace_bytes
    for b in (big, small):
        dev = to_device(b)
        note(f"noalloc case {b.name}: rows={b.num_rows}")
        ref_o, ref_l = run_gpu(b, dev)
        o, l = _noalloc(b, dev)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)
        compare(b, o, l)


@pytest.mark.gpu
def test_noalloc_mixed_config_and_f32():
    """The mixed batch (its 39 MB of partials fit the scratch) and an fp32 batch."""
    for b in (wl.config(4), wl.custom([dict(q_len=3, seq_len=70, q_start=60), dict(q_len=1, seq_len=33)],
                                      hq=4, hkv=2, d=128, dtype="f32", seed=3, num_kv_splits=3)):
        dev = to_device(b)
        note(f"noalloc case {b.name}: rows={b.num_rows}")
        ref_o, ref_l = run_gpu(b, dev)
        o, l = _noalloc(b, dev)
        assert np.array_equal(o, ref_o) and np.array_equal(l, ref_l)


def test_noalloc_refuses_plans_beyond_the_scratch():
    """Host-side check, no GPU: a plan whose tables and partials exceed the
    64 MiB scratch is refused with PMATTN_E_WORKSPACE before any HIP call."""
    import ctypes

    from prefix_shared_paged_pmattn_amd import _lib as L
    n = 64
    bt = np.arange(n * 256, dtype=np.int32).reshape(n, 256)
    p = pm.plan(np.ones(n), np.full(n, 4096), np.full(n, 4095), bt, num_pool_blocks=n * 256, num_q_heads=32,
                num_kv_heads=8, head_dim=128, scale=0.088, num_kv_splits=256)
    assert p.workspace_bytes > 64 << 20
    fake = ctypes.c_void_p(256)   # never dereferenced: the size check comes first
    st = L.load().pmattn_forward_noalloc(p.handle, fake, fake, fake, fake, fake, None, None)
    assert st == L.E_WORKSPACE
    assert "64" in L.load().pmattn_last_error().decode() or "67108864" in L.load().pmattn_last_error().decode()
