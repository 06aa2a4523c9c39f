"""GPU parity at the five workloads' full sizes, on sampled requests.

The HIP path runs exactly as the benchmark launches it (no debug exports); the
oracle recomputes, in fp64, the requests it samples (their target and drafter rows
through the whole head, the Philox uniforms of those request indices) and the
outcomes are compared with the excuse windows. A second call with the debug
exports checks logits (2e-3), probabilities (1e-5) and argmax on the sampled rows.
Drafts for every request are drawn by the oracle from its own fp64 drafter rows.
"""
import numpy as np
import pytest
import torch

import mtp_draft_verification_amd as mv
import oracle
import synth
from gpu_util import TOL_LOGIT, TOL_PROB, WINDOW, compare_outcomes, decode, dev, to_dev

pytestmark = pytest.mark.gpu

# workload id -> (modes, requests the oracle checks)
CASES = {2: (("greedy",), [0]), 3: (("sample",), [0, 5, 13, 31]), 4: (("greedy", "sample"), [0, 21, 42, 63]),
         5: (("sample",), [0, 77, 160, 255])}


@pytest.fixture(scope="module")
def loaded():
    return {}


def _load(cache, cid):
    if cid not in cache:
        cache.clear()  # keep one head at a time in host memory
        wl = synth.WORKLOADS[cid]
        print(f"loading workload {wl.name}", flush=True)
        W_store = synth.weights(wl)
        W64 = decode(W_store, wl.dtype)
        cache[cid] = (wl, to_dev(W_store, wl.dtype), W64)
    return cache[cid]


def _inputs(wl, W64, step):
    xt, xd = synth.hidden(wl, step)
    Xt, Xd = decode(xt, wl.dtype), decode(xd, wl.dtype)
    drafts, _ = oracle.draft_from_hidden(Xd, W64, wl.T, wl.seed, step)
    return xt, xd, Xt, Xd, drafts


def _oracle_requests(wl, mode, Xt, Xd, W64, drafts, step, reqs):
    """Oracle outcomes of the sampled requests, stacked as one batch."""
    outs = []
    for b in reqs:
        if mode == "greedy":
            r = oracle.verify_greedy_from_hidden(Xt[b:b + 1], W64, drafts[b:b + 1])
        else:
            r = oracle.verify_sample_from_hidden(Xt[b:b + 1], Xd[b:b + 1], W64, drafts[b:b + 1], wl.T, wl.seed,
                                                 step, b0=b)
        outs.append(r)
    keys = ["a", "out", "top2_gap"] if mode == "greedy" else ["a", "out", "p_d", "q_d", "u_acc", "u_res", "cdf_lo",
                                                              "cdf_hi"]
    res = {key: np.concatenate([o[key] for o in outs], axis=0) for key in keys}
    res["Lt"] = np.concatenate([o["Lt"] for o in outs], axis=0)
    if mode == "sample":
        res["Ld"] = np.concatenate([o["Ld"] for o in outs], axis=0)
        res["P"] = np.concatenate([o["P"] for o in outs], axis=0)
        res["Q"] = np.concatenate([o["Q"] for o in outs], axis=0)
    return res


def _gpu_call(wl, mode, Wd, xt_d, xd_d, drafts_d, step, debug=None):
    B, k = wl.B, wl.k
    alen = torch.full((B,), -7, dtype=torch.int32, device=dev())
    out = torch.full((B, k + 1), -7, dtype=torch.int32, device=dev())
    ws = mv.alloc_workspace(mv.MODE_GREEDY if mode == "greedy" else mv.MODE_SAMPLE, B, k, wl.H, wl.V,
                            mv.DTYPE_BF16, dev())
    if mode == "greedy":
        mv.spec_verify_greedy(xt_d, Wd, drafts_d, alen, out, ws, debug=debug)
    else:
        mv.spec_verify_sample(xt_d, xd_d, Wd, drafts_d, wl.T, wl.seed, step, alen, out, ws, debug=debug)
    err = mv.get_device_error(ws)
    torch.cuda.synchronize()
    return alen.cpu().numpy(), out.cpu().numpy(), err


@pytest.mark.parametrize("cid,mode", [(c, m) for c, (ms, _) in CASES.items() for m in ms])
def test_fullsize_parity(cid, mode, loaded):
    wl, Wd, W64 = _load(loaded, cid)
    reqs = CASES[cid][1]
    step = 0
    print(f"full-size {wl.name} {mode}: requests {reqs}", flush=True)
    xt, xd, Xt, Xd, drafts = _inputs(wl, W64, step)
    xt_d, xd_d = to_dev(xt, wl.dtype), to_dev(xd, wl.dtype)
    drafts_d = torch.from_numpy(np.ascontiguousarray(drafts)).to(dev())

    # 1) the benchmark's launch configuration: outcomes only
    a, out, err = _gpu_call(wl, mode, Wd, xt_d, xd_d, drafts_d, step)
    assert err == 0
    k = wl.k
    assert np.all((a >= 0) & (a <= k))
    for b in range(wl.B):
        assert np.array_equal(out[b, : a[b]], drafts[b, : a[b]])
        assert np.all(out[b, a[b] + 1:] == -1) and 0 <= out[b, a[b]] < wl.V
    ora = _oracle_requests(wl, mode, Xt, Xd, W64, drafts, step, reqs)
    n, excused, fails = compare_outcomes(mode, {"a": a[reqs], "out": out[reqs]}, ora, k)
    assert not fails, fails
    assert excused <= 1, excused
    print(f"  positions {n} excused {excused}", flush=True)

    # 2) numerics of the sampled rows through the debug exports
    meff = wl.M_eff(mode)
    logits = torch.empty(meff, wl.V, dtype=torch.float32, device=dev())
    probs = torch.empty(meff, wl.V, dtype=torch.float32, device=dev())
    argmax = torch.empty(meff, dtype=torch.int32, device=dev())
    dbg = mv.make_debug(logits=logits, probs=probs, argmax=argmax)
    a2, out2, _ = _gpu_call(wl, mode, Wd, xt_d, xd_d, drafts_d, step, debug=dbg)
    assert np.array_equal(a2, a) and np.array_equal(out2, out)  # exports do not change outcomes
    rows_t = np.array([b * (k + 1) + j for b in reqs for j in range(k + 1)])
    L_gpu = logits[torch.from_numpy(rows_t).to(dev())].cpu().numpy().astype(np.float64)
    L_ora = ora["Lt"].reshape(-1, wl.V)
    assert np.max(np.abs(L_gpu - L_ora)) <= TOL_LOGIT
    P_gpu = probs[torch.from_numpy(rows_t).to(dev())].cpu().numpy().astype(np.float64)
    P_ora = oracle.softmax(L_ora, 1.0 if mode == "greedy" else wl.T)
    assert np.max(np.abs(P_gpu - P_ora)) <= TOL_PROB
    g = np.argmax(L_ora, axis=-1)
    top2 = np.sort(L_ora, axis=-1)[:, -2:]
    am = argmax[torch.from_numpy(rows_t).to(dev())].cpu().numpy()
    assert not np.any((am != g) & (top2[:, 1] - top2[:, 0] > WINDOW))
    if mode == "sample":
        rows_d = np.array([wl.M_t + b * k + j for b in reqs for j in range(k)])
        Ld_gpu = logits[torch.from_numpy(rows_d).to(dev())].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(Ld_gpu - ora["Ld"].reshape(-1, wl.V))) <= TOL_LOGIT
    print(f"  max|dlogit| {np.max(np.abs(L_gpu - L_ora)):.2e} max|dprob| {np.max(np.abs(P_gpu - P_ora)):.2e}",
          flush=True)
