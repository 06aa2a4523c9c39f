"""GPU parity of the MTP input fusion (mtp_input_fuse) against the oracle.

Tolerance, from the arithmetic: the fused input is rounded to bf16 (relative error
at most 2^-9 per element) after fp32 normalization, and the projection accumulates
in fp32 over 2H terms (at most 2H * 2^-24 relative to the sum of magnitudes, far
less in practice). So for every output
  |out_gpu - out_oracle| <= 2^-8 * sum_i |x_i| |W_fc[n, i]| + 1e-6,
with x the oracle's (exact) fused input; and over all outputs the RMS of the error,
each divided by sqrt(sum_i x_i^2 W_fc[n, i]^2), stays below 3e-3 (rounding alone
gives about 2^-9 / sqrt(3) = 1.1e-3; a 10 % error in a norm weight gives ~0.1). Shapes cover the streaming kernel (B <= 3 at
this width) and the tiled kernel, hidden widths with a ragged 256-row tail, a token
out of range (zero embedding half, device error bit) and the Qwen-like width H = 5120.
"""
import numpy as np
import pytest
import torch

import mtp_draft_verification_amd as mv
import oracle
import synth
from gpu_util import dev

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
    bound = 2.0 ** -8 * (np.abs(x) @ np.abs(Wd).T) + 1e-6
    got = out.cpu().numpy().astype(np.float64)
    # statistical check: bf16 rounding of the input gives each output an error of
    # standard deviation about 2^-9 / sqrt(3) * sqrt(sum_i x_i^2 W_ni^2)
    scale = np.sqrt((x * x) @ (Wd * Wd).T) + 1e-12
    assert np.sqrt(np.mean(((got - y) / scale) ** 2)) <= 3e-3
    return got, y, bound, err


@pytest.mark.parametrize("H,V,B", [(256, 1000, 1), (256, 1000, 3), (264, 700, 5), (512, 3000, 40), (1000, 500, 130)])
def test_fuse_parity(H, V, B):
    for step in range(2):
        print(f"fuse H={H} V={V} B={B} step {step}", flush=True)
        got, y, bound, err = _run(H, V, B, step)
        assert err == 0
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - y) <= bound), float(np.max(np.abs(got - y) / bound))


def test_fuse_bad_token_gives_zero_embedding():
    got, y, bound, err = _run(256, 1000, 6, 0, bad=[(1, -4), (4, 1000)])
    assert err == mv.DEVERR_TOKEN_RANGE
    assert np.all(np.abs(got - y) <= bound)
    # and a clean call clears the error word
    assert _run(256, 1000, 6, 1)[3] == 0


def test_fuse_qwen_width():
    """H = 5120 (the batched and depth-5 workloads' width), 32 requests; the table has
    4096 rows (its size only matters to the gather)."""
    got, y, bound, err = _run(5120, 4096, 32, 0)
    assert err == 0
    assert np.all(np.abs(got - y) <= bound), float(np.max(np.abs(got - y) / bound))
