"""Pins of the oracle's MTP input fusion (RMS normalization, concatenation, fc).

* the normalization equals torch.nn.functional.rms_norm (a library routine) in fp64;
* scale invariance with eps = 0: multiplying the hidden state or the embedding row by
  c > 0 leaves its half of the fused input unchanged, and each half has RMS equal to
  the RMS of its weight when the weight is constant;
* the fc product equals math.fsum dot products on sampled entries;
* the halves are in the order [embedding, hidden]: an embedding table of zeros gives
  a zero first half only; an out-of-range token gives a zero embedding half.
"""
import math

import numpy as np
import torch

import oracle


def _inputs(seed, B=5, H=64, V=50):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, V, size=B), rng.normal(size=(V, H)), rng.normal(size=(B, H)) * 3.0,
            rng.normal(1.0, 0.2, size=H), rng.normal(1.0, 0.2, size=H), rng.normal(size=(H, 2 * H)) * 0.05)


def test_rms_norm_matches_torch():
    tok, E, h, ge, gh, W = _inputs(0)
    for eps in (1e-6, 1e-2):
        got = oracle.rms_norm(h, gh, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (h.shape[-1],), torch.from_numpy(gh), eps).numpy()
        assert np.max(np.abs(got - ref)) < 1e-12


def test_scale_invariance_and_unit_rms():
    tok, E, h, ge, gh, W = _inputs(1)
    x1 = oracle.fused_input(tok, E, h, ge, gh, 0.0)
    x2 = oracle.fused_input(tok, E * 7.5, h * 0.01, ge, gh, 0.0)
    assert np.max(np.abs(x1 - x2)) < 1e-12
    H = h.shape[-1]
    x = oracle.fused_input(tok, E, h, np.full(H, 2.0), np.full(H, 0.5), 0.0)
    assert np.allclose(np.sqrt(np.mean(x[:, :H] ** 2, axis=-1)), 2.0)
    assert np.allclose(np.sqrt(np.mean(x[:, H:] ** 2, axis=-1)), 0.5)


def test_fc_matches_fsum():
    tok, E, h, ge, gh, W = _inputs(2)
    y, x = oracle.mtp_input_fuse(tok, E, h, ge, gh, W, 1e-6)
    rng = np.random.default_rng(3)
    for _ in range(20):
        b, n = rng.integers(0, y.shape[0]), rng.integers(0, y.shape[1])
        ref = math.fsum(float(x[b, i]) * float(W[n, i]) for i in range(x.shape[1]))
        assert abs(y[b, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_half_order_and_bad_tokens():
    tok, E, h, ge, gh, W = _inputs(4)
    H = h.shape[-1]
    x = oracle.fused_input(tok, np.zeros_like(E), h, ge, gh, 1e-6)
    assert np.all(x[:, :H] == 0) and np.all(np.abs(x[:, H:]) > 0)
    bad = tok.copy()
    bad[0], bad[1] = -1, E.shape[0]
    xb = oracle.fused_input(bad, E, h, ge, gh, 1e-6)
    assert np.all(xb[:2, :H] == 0)
    assert np.array_equal(xb[2:], oracle.fused_input(tok, E, h, ge, gh, 1e-6)[2:])
