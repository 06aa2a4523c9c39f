"""The allocation-free greedy entry point (spec_verify_greedy_noalloc) against
spec_verify_greedy, through the C ABI: two calls in a row on the one per-GPU scratch
array, the second with a smaller input (a different LM-head kernel and a smaller
workspace layout), every integer output bit-exact, the device error word through the
optional output, and the outcomes also against the oracle.
"""
import numpy as np
import pytest
import torch

import mtp_draft_verification_amd as mv
import oracle
import synth
from gpu_util import compare_outcomes, decode, dev, to_dev

pytestmark = pytest.mark.gpu


def _inputs(wl, step, Wd, W64, bad_draft=False):
    xt, _ = synth.hidden(wl, step)
    Xt = decode(xt, wl.dtype)
    g = np.argmax(oracle.lm_head_logits(Xt, W64), axis=-1)      # [B, k+1], oracle's argmax
    rng = np.random.default_rng(1000 + step)
    drafts = rng.integers(0, wl.V, size=(wl.B, wl.k)).astype(np.int32)
    # half of the requests draft the target's argmax for a random number of slots
    for b in range(0, wl.B, 2):
        n = int(rng.integers(0, wl.k + 1))
        drafts[b, :n] = g[b, :n]
    if bad_draft:
        drafts[0, 0] = wl.V + 3
    return xt, Xt, drafts


def _both(wl, Wd, xt, drafts):
    B, k = wl.B, wl.k
    xt_d = to_dev(xt, wl.dtype)
    d_d = torch.from_numpy(drafts).to(dev())
    a1 = torch.full((B,), -7, dtype=torch.int32, device=dev())
    o1 = torch.full((B, k + 1), -7, dtype=torch.int32, device=dev())
    e1 = torch.full((1,), -7, dtype=torch.int32, device=dev())
    mv.spec_verify_greedy_noalloc(xt_d, Wd, d_d, a1, o1, device_error=e1)
    a2 = torch.full((B,), -9, dtype=torch.int32, device=dev())
    o2 = torch.full((B, k + 1), -9, dtype=torch.int32, device=dev())
    ws = mv.alloc_workspace(mv.MODE_GREEDY, B, k, wl.H, wl.V, mv.DTYPE_BF16, dev())
    mv.spec_verify_greedy(xt_d, Wd, d_d, a2, o2, ws)
    e2 = mv.get_device_error(ws)
    torch.cuda.synchronize()
    return (a1.cpu().numpy(), o1.cpu().numpy(), int(e1.item())), (a2.cpu().numpy(), o2.cpu().numpy(), e2)


def test_noalloc_matches_greedy_two_calls_second_smaller():
    big = synth.custom(H=1024, V=50000, B=8, k=3, cid=610, name="noalloc_big")      # 32 rows: tiled kernel
    small = synth.custom(H=1024, V=50000, B=1, k=3, cid=610, name="noalloc_small")  # 4 rows: streaming kernel
    W_store = synth.weights(big)
    Wd, W64 = to_dev(W_store, "bf16"), decode(W_store, "bf16")
    assert mv.workspace_bytes(8, 3, 1024, 50000, 0, 0) > mv.workspace_bytes(1, 3, 1024, 50000, 0, 0)
    for i, (wl, bad) in enumerate(((big, True), (small, False))):
        print(f"noalloc call {i}: B={wl.B} k={wl.k} H={wl.H} V={wl.V} bad_draft={bad}", flush=True)
        xt, Xt, drafts = _inputs(wl, i, Wd, W64, bad_draft=bad)
        (a1, o1, e1), (a2, o2, e2) = _both(wl, Wd, xt, drafts)
        assert np.array_equal(a1, a2) and np.array_equal(o1, o2)
        assert e1 == e2 == (mv.DEVERR_DRAFT_RANGE if bad else 0)
        ora = oracle.verify_greedy_from_hidden(Xt, W64, drafts)
        n, excused, fails = compare_outcomes("greedy", {"a": a1, "out": o1}, ora, wl.k)
        assert not fails and excused == 0, (fails, excused)
        assert a1.max() > 0 or wl.B == 1
        print(f"  accepted_len {a1.tolist()}", flush=True)


def test_noalloc_without_error_output_and_repeated():
    """device_error = NULL; three calls in a row on one shape give the same outputs."""
    wl = synth.custom(H=512, V=3000, B=5, k=2, cid=611, name="noalloc_rep")
    W_store = synth.weights(wl)
    Wd, W64 = to_dev(W_store, "bf16"), decode(W_store, "bf16")
    xt, Xt, drafts = _inputs(wl, 0, Wd, W64)
    xt_d = to_dev(xt, "bf16")
    d_d = torch.from_numpy(drafts).to(dev())
    outs = []
    for _ in range(3):
        a = torch.full((wl.B,), -7, dtype=torch.int32, device=dev())
        o = torch.full((wl.B, wl.k + 1), -7, dtype=torch.int32, device=dev())
        mv.spec_verify_greedy_noalloc(xt_d, Wd, d_d, a, o)
        torch.cuda.synchronize()
        outs.append((a.cpu().numpy(), o.cpu().numpy()))
    ora = oracle.verify_greedy_from_hidden(Xt, W64, drafts)
    for a, o in outs:
        assert np.array_equal(a, ora["a"]) and np.array_equal(o, ora["out"])
