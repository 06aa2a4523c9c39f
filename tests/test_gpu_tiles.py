"""GPU parity of the LM-head kernels' partial position tiles against the oracle.

The tiled kernel runs a stage loop per count of live 16-position fragments in a
wave's half of a position tile (the rest of the tile is padding whose products are
not formed); the streaming kernel lets the lanes of missing positions in a group of
four read the last position's row. These cases put the last position at every
fragment boundary of each tile height (64, 128 and 256 positions per tile, so 0 to
2, 1 to 4 and 1 to 8 live fragments in the second half) and every partial group of
four on the streaming kernel, with a ragged vocabulary (V % 4 != 0) and, for the
streaming kernel, a ragged hidden width (H not a whole number of 256-byte steps).
Greedy verification, one step each: logits, argmax, accepted lengths and emitted
tokens element by element against the oracle, under the parity tests' rule. Also:
the timing hooks at an interval time one call in n.
"""
import pytest
import torch

import mtp_draft_verification_amd as mv
import synth
from gpu_util import (EXCUSE_RATE, Case, check_invariants, check_numerics, compare_outcomes, gpu_run,
                      load_workload, oracle_run)

pytestmark = pytest.mark.gpu

# greedy, k = 3: M_eff = 4 B head rows
TILED_B = [6, 9, 15,                           # 64 per tile: 0, 1, 2 live fragments in the second half
           17, 21, 25, 29,                     # 128 per tile: 1 .. 4
           33, 37, 41, 45, 49, 53, 57, 61]     # 256 per tile: 1 .. 8
# k = 0: M_eff = B rows on the streaming kernel (partial groups of four)
STREAM_B = [1, 2, 3, 5, 6, 7, 9, 10, 11, 13, 14, 15]


@pytest.fixture(scope="module")
def heads():
    return {}


def _head(cache, wl):
    key = (wl.H, wl.V, wl.cid)
    if key not in cache:
        cache[key] = load_workload(wl)
    return cache[key]


def _check(wl, cache):
    W_store, W64 = _head(cache, wl)
    case = Case(wl, W_store, W64, 0)
    res = gpu_run(case, "greedy")
    ora = oracle_run(case, "greedy")
    assert res["err"] == 0
    check_invariants(res, case.drafts, wl.k)
    check_numerics(res, ora, "greedy", wl)
    n, e, fails = compare_outcomes("greedy", res, ora, wl.k)
    assert not fails, fails
    assert e <= EXCUSE_RATE * n + 1, (e, n)


@pytest.mark.parametrize("B", TILED_B)
def test_partial_position_tiles(B, heads):
    wl = synth.custom(H=256, V=3001, B=B, k=3, cid=170)
    print(f"tiles B={B} M_eff={4 * B} H={wl.H} V={wl.V}", flush=True)
    _check(wl, heads)


@pytest.mark.parametrize("B", STREAM_B)
def test_partial_position_groups(B, heads):
    wl = synth.custom(H=264, V=1001, B=B, k=0, cid=171)
    print(f"groups B={B} M_eff={B} H={wl.H} V={wl.V}", flush=True)
    _check(wl, heads)


def test_timing_hooks_time_one_call_in_n(heads):
    """With the hooks on at an interval of 4, ten verify calls time calls 1, 5 and 9:
    three LM-head launches, each with a positive duration."""
    wl = synth.custom(H=256, V=3001, B=6, k=3, cid=170)
    W_store, W64 = _head(heads, wl)
    case = Case(wl, W_store, W64, 0)
    gpu_run(case, "greedy")  # warm: plan, workspace, first launch
    mv.timing_enable(True, every=4)
    mv.timing_read(reset=True)
    for _ in range(10):
        gpu_run(case, "greedy", debug=False)
    torch.cuda.synchronize()
    ms, n = mv.timing_read(reset=True)
    mv.timing_enable(False)
    assert n == 3, n
    assert ms > 0.0
