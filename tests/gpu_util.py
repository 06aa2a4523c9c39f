"""Shared pieces of the GPU parity tests: seeded inputs for both sides, one call
of the HIP path through the C ABI with its debug exports, one oracle run, and
the comparison rules.

Comparison rules (tolerances of the verify step):
  * logits: max |gpu - oracle| <= 2e-3 (fp32 accumulation against fp64);
  * probabilities: max |gpu - oracle| <= 1e-5;
  * integers (argmax, accepted_len, out_tokens) bit-exact, except a differing
    decision the oracle places inside a window, which is excused and counted:
      greedy argmax: the two largest fp64 logits of that row are within 1e-5;
      acceptance: |u - p(d)/q(d)| <= 1e-5;
      inverse CDF: the uniform is within 1e-5 of an edge of the oracle's token's
      normalised CDF interval.
    After an excused difference the rest of that request is not compared.
    Excused differences must stay below 0.1 % of verified positions.
"""
import numpy as np
import torch

import mtp_draft_verification_amd as mv
import oracle
import synth

TOL_LOGIT = 2e-3
TOL_PROB = 1e-5
WINDOW = 1e-5
EXCUSE_RATE = 1e-3


def dev():
    return torch.device("cuda:0")


def decode(arr, dtype):
    return oracle.decode_bf16(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float64)


def to_dev(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev())


class Case:
    """Inputs of one workload step on both sides. Drafts are drawn by the oracle
    from its own fp64 drafter distribution (Philox word 2 of the verify seed)."""

    def __init__(self, wl, W_store, W64, step, Wd=None):
        self.wl, self.step = wl, step
        xt, xd = synth.hidden(wl, step)
        self.Xt, self.Xd = decode(xt, wl.dtype), decode(xd, wl.dtype)
        self.W64 = W64
        if wl.k > 0:
            self.drafts, _ = oracle.draft_from_hidden(self.Xd, W64, wl.T, wl.seed, step)
        else:
            self.drafts = np.zeros((wl.B, 0), dtype=np.int32)
        self.xt_d, self.xd_d = to_dev(xt, wl.dtype), to_dev(xd, wl.dtype)
        self.W_d = Wd if Wd is not None else to_dev(W_store, wl.dtype)
        self.drafts_d = torch.from_numpy(np.ascontiguousarray(self.drafts, dtype=np.int32)).to(dev())


def load_workload(wl):
    W_store = synth.weights(wl)
    return W_store, decode(W_store, wl.dtype)


def gpu_run(case, mode, drafts_d=None, xd_d=None, debug=True):
    """One verify call through the C ABI; returns numpy outputs and debug exports."""
    wl = case.wl
    B, k, V = wl.B, wl.k, wl.V
    drafts_d = case.drafts_d if drafts_d is None else drafts_d
    xd_d = case.xd_d if xd_d is None else xd_d
    meff = B * (k + 1) + (B * k if mode == "sample" else 0)
    d = dev()
    alen = torch.full((B,), -7, dtype=torch.int32, device=d)
    out = torch.full((B, k + 1), -7, dtype=torch.int32, device=d)
    code = mv.DTYPE_BF16 if wl.dtype == "bf16" else mv.DTYPE_F32
    ws = mv.alloc_workspace(mv.MODE_GREEDY if mode == "greedy" else mv.MODE_SAMPLE, B, k, wl.H, V, code, d)
    ex = {}
    dbg = None
    if debug:
        ex = dict(logits=torch.empty(meff, V, dtype=torch.float32, device=d),
                  probs=torch.empty(meff, V, dtype=torch.float32, device=d),
                  argmax=torch.empty(meff, dtype=torch.int32, device=d),
                  row_stats=torch.empty(meff, 2, dtype=torch.float64, device=d),
                  pd_qd=torch.empty(max(B * k, 1), 2, dtype=torch.float64, device=d))
        dbg = mv.make_debug(**ex)
    if mode == "greedy":
        mv.spec_verify_greedy(case.xt_d, case.W_d, drafts_d, alen, out, ws, debug=dbg)
    else:
        mv.spec_verify_sample(case.xt_d, xd_d, case.W_d, drafts_d, wl.T, wl.seed, case.step, alen, out, ws,
                              debug=dbg)
    err = mv.get_device_error(ws)
    torch.cuda.synchronize()
    res = {"a": alen.cpu().numpy(), "out": out.cpu().numpy(), "err": err}
    for n, t in ex.items():
        res[n] = t.cpu().numpy()
    return res


def oracle_run(case, mode, drafts=None, Xd=None):
    wl = case.wl
    drafts = case.drafts if drafts is None else drafts
    Xd = case.Xd if Xd is None else Xd
    if mode == "greedy":
        return oracle.verify_greedy_from_hidden(case.Xt, case.W64, drafts)
    return oracle.verify_sample_from_hidden(case.Xt, Xd, case.W64, drafts, wl.T, wl.seed, case.step)


def check_invariants(res, drafts, k):
    a, out = res["a"], res["out"]
    assert np.all((a >= 0) & (a <= k))
    for b in range(len(a)):
        assert np.array_equal(out[b, : a[b]], drafts[b, : a[b]])
        assert np.all(out[b, a[b] + 1:] == -1)
        assert out[b, a[b]] >= 0


def compare_outcomes(mode, res, ora, k, details=None):
    """Returns (positions, excused, failing requests). With a list `details`, appends
    (request, window, distance to the threshold) for every excused difference."""
    a_g, out_g = res["a"], res["out"]
    a_o, out_o = ora["a"], ora["out"]
    B = len(a_g)
    excused, fails = 0, []
    for b in range(B):
        if a_g[b] == a_o[b] and np.array_equal(out_g[b], out_o[b]):
            continue
        j = int(min(a_g[b], a_o[b]))
        if mode == "greedy":
            kind, dist = "argmax", float(ora["top2_gap"][b, j])
        elif a_g[b] != a_o[b]:
            pd, qd = ora["p_d"][b, j], ora["q_d"][b, j]
            ratio = pd / qd if qd > 0 else np.inf
            kind, dist = "accept", float(abs(ora["u_acc"][b, j] - ratio))
        else:
            u = ora["u_res"][b]
            kind, dist = "cdf", float(min(abs(u - ora["cdf_lo"][b]), abs(u - ora["cdf_hi"][b])))
        if dist <= WINDOW:
            excused += 1
            if details is not None:
                details.append((b, kind, dist))
        else:
            fails.append((b, int(a_g[b]), int(a_o[b]), out_g[b].tolist(), out_o[b].tolist()))
    return B * (k + 1), excused, fails


def oracle_probs(ora, mode, T):
    if mode == "greedy":
        return oracle.softmax(ora["Lt"], 1.0).reshape(-1, ora["Lt"].shape[-1])
    P = ora["P"].reshape(-1, ora["P"].shape[-1])
    Q = ora["Q"].reshape(-1, ora["Q"].shape[-1])
    return np.concatenate([P, Q], axis=0)


def oracle_logits(ora, mode):
    Lt = ora["Lt"].reshape(-1, ora["Lt"].shape[-1])
    if mode == "greedy":
        return Lt
    return np.concatenate([Lt, ora["Ld"].reshape(-1, ora["Ld"].shape[-1])], axis=0)


def check_numerics(res, ora, mode, wl):
    """Logit and probability tolerances, argmax parity on every row."""
    L = oracle_logits(ora, mode)
    assert res["logits"].shape == L.shape
    err = np.max(np.abs(res["logits"].astype(np.float64) - L))
    assert err <= TOL_LOGIT, err
    P = oracle_probs(ora, mode, wl.T)
    perr = np.max(np.abs(res["probs"].astype(np.float64) - P))
    assert perr <= TOL_PROB, perr
    g = np.argmax(L, axis=-1)
    top2 = np.sort(L, axis=-1)[:, -2:] if L.shape[-1] > 1 else np.zeros((L.shape[0], 2))
    gap = top2[:, 1] - top2[:, 0]
    bad = (res["argmax"] != g) & (gap > WINDOW)
    assert not np.any(bad), np.nonzero(bad)
    return err, perr
