"""GPU parity of the top-k soft cross-entropy draft loss (mtp_draft_loss_topk) against
the oracle, through the C ABI.

The kept token ids must match the oracle exactly (fp32 comparisons on both sides,
ties to the lower id). Losses and gradients are floating point; their tolerances
follow from the kernel's arithmetic:

* loss: the student normalizer sums 2^((s - m) log2 e) terms from the hardware exp2
  (the fp32 product's rounding gives <= |s - m| * 1e-7 relative error, so <= ~5e-7 on
  the terms that carry the sum), in fp32 groups of 4 accumulated in fp64, so
  logsumexp is off by <= ~5e-7; the soft targets and the gathered dot product are
  fp64; the result is rounded to fp32. Bound used: |d loss| <= 2e-6 + 1e-6 |loss|.
* gradient: q = expf(float(s - lse)); the fp32 rounding of the exponent argument
  (|s - lse| <= ~40) moves q by <= ~2e-6 relative, lse by <= 5e-7, expf by 2 ulp;
  the fp32 result adds half an ulp. Bound used:
  |d g| <= scale * 4e-6 * q_ref + 1.2e-7 |g_ref| + 1e-30.

Shapes: 16-byte path (V % 4 == 0) and 4-byte path (V odd), many equal teacher
logits at the cut, k = 1, k = 512 (the maximum) and k = V, a vocabulary smaller than
one pass of the workgroup, rows whose teacher logits ascend (every token enters the
kept buffers, which are cut again and again), and the full benchmark launch
(4096 rows x 151936 tokens, k = 256) with every row checked: the rows repeat 8
seeded rows, so each output has an oracle value.
"""
import numpy as np
import pytest
import torch

import mtp_draft_verification_amd as mv
import oracle
import synth

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def run_gpu(T, S, k, scale=None, want_grad=False):
    N, V = T.shape
    Td = torch.from_numpy(np.ascontiguousarray(T)).to(dev())
    Sd = torch.from_numpy(np.ascontiguousarray(S)).to(dev())
    loss = torch.full((N,), float("nan"), dtype=torch.float32, device=dev())
    idx = torch.full((N, k), -7, dtype=torch.int32, device=dev())
    grad = torch.full((N, V), float("nan"), dtype=torch.float32, device=dev()) if want_grad else None
    ws = mv.alloc_loss_workspace(N, k, dev())
    mv.mtp_draft_loss_topk(Td, Sd, k, loss, ws, 1.0 if scale is None else scale, idx, grad)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), idx.cpu().numpy(), (grad.cpu().numpy() if want_grad else None)


def check_rows(T, S, k, loss, idx, grad=None, scale=1.0, rows=None):
    rows = range(T.shape[0]) if rows is None else rows
    for n in rows:
        ref, K, pt, lse = oracle.draft_loss_row(T[n], S[n], k)
        assert np.array_equal(idx[n], K), (n, idx[n][:8], K[:8])
        assert abs(loss[n] - ref) <= 2e-6 + 1e-6 * abs(ref), (n, loss[n], ref)
        if grad is not None:
            q = np.exp(S[n].astype(np.float64) - lse)
            g = scale * q
            g[K] -= scale * pt
            tol = scale * 4e-6 * q + 1.2e-7 * np.abs(g) + 1e-30
            bad = np.abs(grad[n] - g) > tol
            assert not bad.any(), (n, np.flatnonzero(bad)[:5], grad[n][bad][:5], g[bad][:5])


@pytest.mark.parametrize("V", [3000, 2999])
def test_small_rows_with_gradient(V):
    print(f"loss small V={V}", flush=True)
    T, S = synth.loss_rows(V, range(6), cid=410 + V % 2)
    loss, idx, grad = run_gpu(T, S, 256, scale=0.37, want_grad=True)
    check_rows(T, S, 256, loss, idx, grad, scale=0.37)


def test_equal_logits_at_the_cut():
    print("loss ties", flush=True)
    T, S = synth.loss_rows(5000, range(4), cid=412, quantum=0.5)
    loss, idx, grad = run_gpu(T, S, 256, want_grad=True)
    check_rows(T, S, 256, loss, idx, grad)


@pytest.mark.parametrize("k,V", [(1, 4096), (512, 40000), (300, 300), (5, 37)])
def test_k_extremes(k, V):
    print(f"loss k={k} V={V}", flush=True)
    T, S = synth.loss_rows(V, range(3), cid=413)
    loss, idx, grad = run_gpu(T, S, k, want_grad=True)
    check_rows(T, S, k, loss, idx, grad)


@pytest.mark.parametrize("k", [256, 512])
def test_ascending_teacher_rows(k):
    """Every token beats the running threshold: the buffers are cut on every few passes."""
    print(f"loss ascending k={k}", flush=True)
    V = 20000
    T, S = synth.loss_rows(V, range(2), cid=414)
    T = np.sort(T, axis=1)
    T[1] = T[1][::-1].copy()            # and one descending row (nothing enters after the first pass)
    loss, idx, _ = run_gpu(T, S, k)
    check_rows(T, S, k, loss, idx)


def test_many_rows_with_random_teacher_order():
    print("loss 64 rows V=50000", flush=True)
    T, S = synth.loss_rows(50000, range(64), cid=415)
    loss, idx, _ = run_gpu(T, S, 256)
    check_rows(T, S, 256, loss, idx)


def test_full_size_launch_every_row():
    """The benchmark's launch: 4096 rows x 151936 tokens, k = 256, with the gradient."""
    N, V, k, P = 4096, 151936, 256, 8
    print(f"loss full size N={N} V={V} k={k}", flush=True)
    T8, S8 = synth.loss_rows(V, range(P), cid=416)
    refs = [oracle.draft_loss_row(T8[i], S8[i], k) for i in range(P)]
    Td = torch.from_numpy(T8).to(dev()).repeat(N // P, 1).contiguous()
    Sd = torch.from_numpy(S8).to(dev()).repeat(N // P, 1).contiguous()
    loss = torch.full((N,), float("nan"), dtype=torch.float32, device=dev())
    idx = torch.full((N, k), -7, dtype=torch.int32, device=dev())
    grad = torch.full((N, V), float("nan"), dtype=torch.float32, device=dev())
    ws = mv.alloc_loss_workspace(N, k, dev())
    scale = 1.0 / N
    mv.mtp_draft_loss_topk(Td, Sd, k, loss, ws, scale, idx, grad)
    torch.cuda.synchronize()
    loss_h, idx_h = loss.cpu().numpy(), idx.cpu().numpy()
    for n in range(N):
        ref, K, _, _ = refs[n % P]
        assert np.array_equal(idx_h[n], K), n
        assert abs(loss_h[n] - ref) <= 2e-6 + 1e-6 * abs(ref), (n, loss_h[n], ref)
    # gradient rows: every position of a sample of rows (all 8 patterns)
    for n in [0, 1, 2, 3, 4, 5, 6, 7, 1234, 4095]:
        _, K, pt, lse = refs[n % P]
        q = np.exp(S8[n % P].astype(np.float64) - lse)
        g = scale * q
        g[K] -= scale * pt
        got = grad[n].cpu().numpy()
        tol = scale * 4e-6 * q + 1.2e-7 * np.abs(g) + 1e-30
        assert not (np.abs(got - g) > tol).any(), n
    # and the whole gradient: finite, each row sums to ~0
    rs = grad.double().sum(dim=1).abs().max().item()
    assert torch.isfinite(grad).all().item() and rs <= 1e-6 * scale * 100, rs
