"""Token-budget batch builder (include/pmattn_batch.h) against its Python
restatement, plus the properties the pages ask of a step (XY-Serve review,
Figure 6 caption): never above the budget, prefill never in the reserved
slots, decode/verify rows never split."""
import numpy as np
import pytest

import prefix_shared_paged_pmattn_amd as pm
from oracle import plan_replica as R
from prefix_shared_paged_pmattn_amd import _lib


@pytest.mark.parametrize("seed", range(8))
def test_matches_replica_and_invariants(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(rng.integers(0, 200))
    kinds = rng.integers(0, 3, size=n)
    context = rng.integers(0, 8000, size=n)
    pending = np.where(kinds == 1, 1, np.where(kinds == 2, rng.integers(1, 9, size=n),
                                               rng.integers(0, 3000, size=n)))
    budget = int(rng.integers(1, 9000))
    reserved = int(rng.integers(0, budget + 1))
    chunk = int(rng.integers(1, 2048))
    q = pm.build_batch(kinds, context, pending, token_budget=budget, reserved=reserved, max_chunk=chunk)
    want = R.build_batch(kinds.tolist(), context.tolist(), pending.tolist(), budget, reserved, chunk)
    assert np.array_equal(q, want)
    pre = kinds == 0
    assert q.sum() <= budget and q[pre].sum() <= budget - reserved
    assert ((q[~pre] == 0) | (q[~pre] == pending[~pre])).all()       # decode/verify whole or not at all
    assert (q[pre] <= np.minimum(pending[pre], chunk)).all()
    # prefills complete in order: after the first prefill that got less than it wanted, none gets rows
    short = np.nonzero(pre & (q < np.minimum(pending, chunk)) & (pending > 0))[0]
    if short.size:
        later = np.arange(n) > short[0]
        assert (q[later & pre] == 0).all()


def test_mixed_step_of_the_pages_shape():
    """16 long prompts, 96 decodes and 32 five-draft verifies under a 8,448-row
    budget with 256 rows reserved and 512-row chunks: the step holds 16 x 512
    prefill rows, every decode and every verify (the mixed-chunk workload)."""
    kinds = [0] * 16 + [1] * 96 + [2] * 32
    context = list(range(0, 4096, 256)) + [4000] * 96 + [3000] * 32
    pending = [5000] * 16 + [1] * 96 + [5] * 32
    q = pm.build_batch(kinds, context, pending, token_budget=8448, reserved=256, max_chunk=512)
    assert q[:16].tolist() == [512] * 16 and (q[16:112] == 1).all() and (q[112:] == 5).all()
    assert q.sum() == 8448


def test_errors():
    with pytest.raises(pm.PmattnError):
        pm.build_batch([1], [0], [2], token_budget=10, reserved=0, max_chunk=4)   # decode of 2 rows
    with pytest.raises(pm.PmattnError):
        pm.build_batch([0], [0], [5], token_budget=10, reserved=11, max_chunk=4)
    with pytest.raises(pm.PmattnError):
        pm.build_batch([3], [0], [1], token_budget=10, reserved=0, max_chunk=4)
    assert pm.build_batch([], [], [], token_budget=1, reserved=0, max_chunk=1).shape == (0,)
