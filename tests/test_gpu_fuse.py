"""GPU parity of the MTP input fusion (mtp_input_fuse) against the oracle.

Every output must lie within 2e-3 of the oracle's fp64 result (the verify step's
logit tolerance; the fc output feeds the drafter the same way the head's output
feeds the verifier). The fused input reaches the bf16 projection as a bf16 hi part
plus a bf16 lo part, so it carries about 17 bits (relative error <= 2^-17 per
element) instead of bf16's 8, and the projection accumulates in fp32; so also the
RMS over all outputs of the error, each divided by sqrt(sum_i x_i^2 W_fc[n, i]^2),
must stay below 1e-4 (the hi/lo residual alone gives about 2^-17 / sqrt(3) = 4.4e-6;
rounding the input to bf16 alone would give 1.1e-3; a 10 % error in a norm weight
gives ~0.1). Shapes cover the streaming kernel (2B <= 3 rows at this width) and the
tiled kernel with its K split (one and several position chunks), hidden widths with
a ragged 256-row tail, a token out of range (zero embedding half, device error bit),
the Qwen-like width H = 5120 and the rollout width H = 7168 with 256 requests.
"""
import numpy as np
import pytest
import torch

import mtp_draft_verification_amd as mv
import oracle
import synth
from gpu_util import TOL_LOGIT, dev

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def _run(H, V, B, step, bad=()):
    tokens, E, h, ge, gh, W = synth.fuse_inputs(H, V, B, cid=300 + H % 97, step=step)
    tokens = tokens.copy()
    for i, t in bad:
        tokens[i] = t
    out = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev())
    ws = mv.alloc_fuse_workspace(B, H, dev())
    mv.mtp_input_fuse(torch.from_numpy(tokens).to(dev()), _bf16_dev(E), _bf16_dev(h), _bf16_dev(ge), _bf16_dev(gh),
                      _bf16_dev(W), 1e-6, out, ws)
    err = mv.get_device_error(ws)
    torch.cuda.synchronize()
    dec = oracle.decode_bf16
    y, x = oracle.mtp_input_fuse(tokens, dec(E), dec(h), dec(ge), dec(gh), dec(W), 1e-6)
    Wd = dec(W)
    got = out.cpu().numpy().astype(np.float64)
    scale = np.sqrt((x * x) @ (Wd * Wd).T) + 1e-12
    rms = float(np.sqrt(np.mean(((got - y) / scale) ** 2)))
    assert rms <= 1e-4, rms
    return got, y, err


@pytest.mark.parametrize("H,V,B", [(256, 1000, 1), (256, 1000, 3), (264, 700, 5), (512, 3000, 40), (1000, 500, 130)])
def test_fuse_parity(H, V, B):
    for step in range(2):
        print(f"fuse H={H} V={V} B={B} step {step}", flush=True)
        got, y, err = _run(H, V, B, step)
        assert err == 0
        assert np.all(np.isfinite(got))
        assert float(np.max(np.abs(got - y))) <= TOL_LOGIT, float(np.max(np.abs(got - y)))


def test_fuse_bad_token_gives_zero_embedding():
    got, y, err = _run(256, 1000, 6, 0, bad=[(1, -4), (4, 1000)])
    assert err == mv.DEVERR_TOKEN_RANGE
    assert float(np.max(np.abs(got - y))) <= TOL_LOGIT
    # and a clean call clears the error word
    assert _run(256, 1000, 6, 1)[2] == 0


def test_fuse_qwen_width():
    """H = 5120 (the batched and depth-5 workloads' width), 32 requests; the table has
    4096 rows (its size only matters to the gather)."""
    got, y, err = _run(5120, 4096, 32, 0)
    assert err == 0
    print(f"H=5120 B=32: max |err| {float(np.max(np.abs(got - y))):.2e}", flush=True)
    assert float(np.max(np.abs(got - y))) <= TOL_LOGIT, float(np.max(np.abs(got - y)))


def test_fuse_rollout_width():
    """H = 7168 with 256 requests (512 fused rows: two position chunks of the K-split
    tiled kernel), and one request at H = 4096 (the streaming kernel)."""
    for H, V, B in ((7168, 2048, 256), (4096, 2048, 1)):
        got, y, err = _run(H, V, B, 0)
        assert err == 0
        print(f"H={H} B={B}: max |err| {float(np.max(np.abs(got - y))):.2e}", flush=True)
        assert float(np.max(np.abs(got - y))) <= TOL_LOGIT, float(np.max(np.abs(got - y)))
