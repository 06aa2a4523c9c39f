"""GPU parity of the tiled LM-head kernel's split tiles, in both tile geometries.

With one position chunk and more whole vocabulary tiles than compute units, the whole
rounds of tiles run as they are and the tiles left over are cut along the hidden
dimension into 2 to 8 pieces that fill the otherwise idle compute units; each piece
writes its raw fp32 accumulators and a second kernel adds the pieces in order and
finishes those tiles (statistics, argmax, draft logits, logits out). The tiled kernel
takes more than 96 head rows; up to 128 rows it uses 192-row x 128-position tiles with
a deeper W ring, above that 256 x 224. These shapes give leftovers of 24, 83, 19, 82
and 121 tiles (pieces capped by 8, by the compute units and by the stage count), with
H a whole number of 64-wide stages and not, V ragged and not, head rows in both
geometries, both modes, over two steps each: logits, probabilities, argmax, p(d) and
q(d), accepted lengths and emitted tokens against the oracle under the parity tests'
rule. Vocabularies of exactly two rounds of whole tiles (nothing split) are the
controls.
"""
import pytest

import synth
from gpu_util import (EXCUSE_RATE, Case, check_invariants, check_numerics, compare_outcomes, gpu_run,
                      load_workload, oracle_run, to_dev)

pytestmark = pytest.mark.gpu

C = synth.custom
# (head, mode, B): greedy verifies B (k + 1) rows, stochastic B (2k + 1); k = 3 throughout.
# Small geometry: 97..128 rows, 192-row tiles (12 fragments), 256 tiles per round.
# Large geometry: 129..224 rows, 256-row tiles (16 fragments).
HEADS = {
    "small_left24": dict(H=320, V=192 * (256 + 24), cid=185),          # 5 stages: 5 pieces
    "small_left83_ragged": dict(H=200, V=192 * (256 + 82) + 7, cid=186),  # H % 64 = 8, V % 16 = 7
    "small_whole": dict(H=192, V=192 * 512, cid=187),
    "large_left82": dict(H=320, V=256 * (256 + 82), cid=180),          # 3 pieces
    "large_left19_ragged_h": dict(H=200, V=70336, cid=181),            # 4 stages: 4 pieces
    "large_left121_ragged": dict(H=136, V=256 * (256 + 120) + 5, cid=182),  # 2 pieces
    "large_whole": dict(H=192, V=256 * 512, cid=184),
}
CASES = [
    ("small_left24", "greedy", 30), ("small_left24", "sample", 16),
    ("small_left83_ragged", "greedy", 26), ("small_left83_ragged", "sample", 15),
    ("small_whole", "greedy", 32),
    ("large_left82", "greedy", 40), ("large_left82", "sample", 32),
    ("large_left19_ragged_h", "greedy", 36), ("large_left19_ragged_h", "sample", 20),
    ("large_left121_ragged", "greedy", 50), ("large_left121_ragged", "sample", 25),
    ("large_whole", "sample", 24),
]
STEPS = 2


@pytest.fixture(scope="module")
def weights_cache():
    return {}


def _weights(cache, wl):
    if wl.cid not in cache:
        cache.clear()  # one head at a time in host memory
        W_store, W64 = load_workload(wl)
        cache[wl.cid] = (W_store, W64, to_dev(W_store, wl.dtype))
    return cache[wl.cid]


@pytest.mark.parametrize("name,mode,B", CASES)
def test_split_tile_parity(name, mode, B, weights_cache):
    wl = C(B=B, k=3, T=0.9, **HEADS[name])
    rows = B * 4 + (B * 3 if mode == "sample" else 0)
    print(f"split {name} mode {mode} H={wl.H} V={wl.V} B={B} rows={rows}", flush=True)
    W_store, W64, Wd = _weights(weights_cache, wl)
    positions = excused = 0
    for step in range(STEPS):
        case = Case(wl, W_store, W64, step, Wd)
        res = gpu_run(case, mode)
        ora = oracle_run(case, mode)
        assert res["err"] == 0
        check_invariants(res, case.drafts, wl.k)
        check_numerics(res, ora, mode, wl)
        n, e, fails = compare_outcomes(mode, res, ora, wl.k)
        assert not fails, fails
        positions += n
        excused += e
    assert excused <= EXCUSE_RATE * positions + (1 if positions < 1000 else 0), (excused, positions)
