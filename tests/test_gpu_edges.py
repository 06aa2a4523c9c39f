"""GPU parity at the edges of the shape space, through the C ABI:

* a one-token vocabulary (V = 1): every distribution is a point mass, so every
  in-range draft is kept and the bonus is token 0;
* the narrowest hidden width (H = 8) and the largest draft count (k = 64);
* many requests: 2000 requests x 4 positions (8000 target rows, 14000 with the
  drafter rows: dozens of position chunks of the tiled kernel);
* the largest call the boundary accepts: M_eff = 65532 head rows (limit 65535).

Outcomes are compared with the oracle with the excuse windows of the other tests.
"""
import numpy as np
import pytest

import synth
from gpu_util import (EXCUSE_RATE, Case, check_invariants, check_numerics, compare_outcomes, gpu_run,
                      load_workload, oracle_run, to_dev)

pytestmark = pytest.mark.gpu

C = synth.custom


def _run_case(wl, mode, steps=1, debug=False):
    W_store, W64 = load_workload(wl)
    Wd = to_dev(W_store, wl.dtype)
    positions = excused = 0
    for step in range(steps):
        print(f"edge {wl.name} {mode} B={wl.B} k={wl.k} H={wl.H} V={wl.V} step {step}", flush=True)
        case = Case(wl, W_store, W64, step, Wd)
        res = gpu_run(case, mode, debug=debug)
        assert res["err"] == 0
        check_invariants(res, case.drafts, wl.k)
        ora = oracle_run(case, mode)
        if debug:
            check_numerics(res, ora, mode, wl)
        n, e, fails = compare_outcomes(mode, res, ora, wl.k)
        assert not fails, fails[:5]
        positions += n
        excused += e
    assert excused <= EXCUSE_RATE * positions + 1, (excused, positions)
    return res


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_one_token_vocabulary(mode):
    wl = C(H=64, V=1, B=4, k=3, cid=140)
    res = _run_case(wl, mode)
    assert np.all(res["a"] == wl.k) and np.all(res["out"] == 0)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_narrowest_hidden(mode):
    _run_case(C(H=8, V=300, B=3, k=2, cid=141), mode, steps=3, debug=True)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_largest_draft_count(mode):
    _run_case(C(H=64, V=500, B=2, k=64, T=0.9, cid=142), mode, steps=2, debug=True)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_many_requests(mode):
    _run_case(C(H=64, V=700, B=2000, k=3, T=0.9, cid=143), mode)


def test_largest_call():
    """16383 requests x 4 target rows = 65532 head rows, greedy."""
    _run_case(C(H=64, V=64, B=16383, k=3, cid=144), "greedy")
