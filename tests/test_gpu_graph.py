"""The verify calls captured in a HIP graph (torch.cuda.CUDAGraph on the current
stream), for callers that replay one step's launches without the host in the loop:
the streaming kernel (greedy, 16 head rows), the tiled kernel (greedy, 132 rows; and
the no-allocation entry point, whose workspace is the library's scratch array), and
the stochastic path with its sampling passes (112 head rows). Each graph is captured
after one eager call (which sets the kernels' LDS limits and the scratch address), then
replayed four times, each time after new seeded inputs are copied into the captured
buffers and with an eager call of the same step run between replays; every replay's
accepted lengths and tokens must equal the eager call's bit for bit, and the replays'
tokens must differ from one another (they read the new inputs). The calls record
no memset and no event (the timing hooks are off), only kernel launches.
"""
import numpy as np
import pytest
import torch

import mtp_draft_verification_amd as mv
import synth
from gpu_util import dev, load_workload, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _inputs(wl, step):
    xt, xd = synth.hidden(wl, step)
    rng = np.random.default_rng(1000 + step)
    drafts = rng.integers(0, wl.V, size=(wl.B, wl.k), dtype=np.int32)
    return to_dev(xt, wl.dtype), to_dev(xd, wl.dtype), torch.from_numpy(drafts).to(dev())


def _run_graph(wl, call):
    """call(xt, xd, drafts, alen, out, step) launches one verify; returns the replays'
    and eager outputs."""
    B, k = wl.B, wl.k
    xt, xd, dr = _inputs(wl, 0)
    alen = torch.full((B,), -7, dtype=torch.int32, device=dev())
    out = torch.full((B, k + 1), -7, dtype=torch.int32, device=dev())
    alen_e, out_e = alen.clone(), out.clone()
    call(xt, xd, dr, alen, out)  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(xt, xd, dr, alen, out)
    torch.cuda.synchronize()
    seen = []
    for r in range(1, REPLAYS + 1):
        nxt, nxd, ndr = _inputs(wl, r)
        xt.copy_(nxt)
        xd.copy_(nxd)
        dr.copy_(ndr)
        alen.fill_(-7)
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(xt, xd, dr, alen_e, out_e)  # eager, same inputs, between replays
        torch.cuda.synchronize()
        np.testing.assert_array_equal(alen.cpu().numpy(), alen_e.cpu().numpy(), err_msg=f"replay {r}")
        np.testing.assert_array_equal(out.cpu().numpy(), out_e.cpu().numpy(), err_msg=f"replay {r}")
        assert int(alen.min()) >= 0
        seen.append(out.cpu().numpy().copy())
    # the replays read the buffers' new contents: their emitted tokens differ
    assert any(not np.array_equal(seen[0], o) for o in seen[1:])
    del g


@pytest.mark.parametrize("B", [4, 33])  # 16 rows: streaming kernel; 132 rows: tiled kernel
def test_greedy_in_graph(B):
    wl = synth.custom(H=256, V=3001, B=B, k=3, cid=174)
    print(f"graph greedy B={B}", flush=True)
    W = to_dev(load_workload(wl)[0], wl.dtype)
    ws = mv.alloc_workspace(mv.MODE_GREEDY, B, wl.k, wl.H, wl.V, mv.DTYPE_BF16, dev())
    _run_graph(wl, lambda xt, xd, dr, a, o: mv.spec_verify_greedy(xt, W, dr, a, o, ws))


def test_noalloc_in_graph():
    wl = synth.custom(H=256, V=3001, B=33, k=3, cid=174)
    print("graph greedy no-alloc B=33", flush=True)
    W = to_dev(load_workload(wl)[0], wl.dtype)
    _run_graph(wl, lambda xt, xd, dr, a, o: mv.spec_verify_greedy_noalloc(xt, W, dr, a, o))


def test_sample_in_graph():
    wl = synth.custom(H=256, V=3001, B=16, k=3, T=0.8, cid=174)
    print("graph sample B=16", flush=True)
    W = to_dev(load_workload(wl)[0], wl.dtype)
    ws = mv.alloc_workspace(mv.MODE_SAMPLE, wl.B, wl.k, wl.H, wl.V, mv.DTYPE_BF16, dev())
    _run_graph(wl, lambda xt, xd, dr, a, o: mv.spec_verify_sample(xt, xd, W, dr, wl.T, wl.seed, 5, a, o, ws))
