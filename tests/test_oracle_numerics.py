"""Pins of the oracle's numerics layer, special cases, invariants and metrics.

* bf16 decoding against torch's own bfloat16 -> float64 conversion;
* the head's logits against math.fsum dot products on sampled entries;
* softmax against scipy.special.softmax;
* k = 0 reduces to plain inverse-transform sampling (numpy searchsorted);
* q = p keeps every draft; V = 1 keeps every draft;
* greedy argmax takes the lowest id on ties; index alignment (p_j judges d[j],
  p_k gives the bonus);
* invariants of every verify outcome (0 <= a <= k, kept prefix = drafts, -1 padding,
  a rejected draft is never its own replacement, residual mass > 0 on rejection);
* the acceptance metrics against the worked example the SkyRL page prints.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import (acceptance_metrics, decode_bf16, greedy_verify, inverse_cdf, lm_head_logits,
                    residual_weights, sample_drafts, softmax, stochastic_verify, verify_uniforms)

HERE = os.path.dirname(os.path.abspath(__file__))


def test_decode_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=50_000, dtype=np.uint64).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]           # drop inf / nan patterns
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(decode_bf16(bits), ref)


def test_logits_match_fsum():
    rng = np.random.default_rng(1)
    X = rng.normal(size=(7, 96))
    W = rng.normal(size=(300, 96))
    L = lm_head_logits(X, W)
    for _ in range(200):
        r, v = rng.integers(7), rng.integers(300)
        exact = math.fsum(float(a) * float(b) for a, b in zip(X[r], W[v]))
        assert abs(L[r, v] - exact) <= 1e-12 * max(1.0, abs(exact))


@pytest.mark.parametrize("T", [0.7, 1.0, 2.5])
def test_softmax_matches_scipy(T):
    rng = np.random.default_rng(2)
    L = rng.normal(size=(5, 1000)) * 4
    np.testing.assert_allclose(softmax(L, T), scipy.special.softmax(L / T, axis=-1), rtol=1e-13, atol=0)


def test_k0_is_inverse_transform_sampling():
    rng = np.random.default_rng(3)
    B, V = 500, 37
    P = softmax(rng.normal(size=(B, 1, V)))
    u_acc, u_res, _ = verify_uniforms(4, 9, B, 0)
    a, out, _ = stochastic_verify(P, np.zeros((B, 0, V)), np.zeros((B, 0), dtype=np.int64), u_acc, u_res)
    assert np.all(a == 0)
    ref = [np.searchsorted(np.cumsum(P[b, 0]), u_res[b, 0] * P[b, 0].sum(), side="right") for b in range(B)]
    assert out[:, 0].tolist() == ref


def test_q_equal_p_keeps_everything_and_V1():
    rng = np.random.default_rng(4)
    B, k, V = 300, 4, 50
    P = softmax(rng.normal(size=(B, k + 1, V)))
    u_acc, u_res, u_draft = verify_uniforms(1, 2, B, k)
    drafts = sample_drafts(P[:, :k], u_draft)
    a, out, _ = stochastic_verify(P, P[:, :k].copy(), drafts, u_acc, u_res)
    assert np.all(a == k)
    assert np.array_equal(out[:, :k], drafts)
    ones = np.ones((B, k + 1, 1))
    a, out, _ = stochastic_verify(ones, ones[:, :k], np.zeros((B, k), dtype=np.int64), u_acc, u_res)
    assert np.all(a == k) and np.all(out == 0)


def test_greedy_ties_and_alignment():
    V = 6
    Lt = np.zeros((1, 3, V))
    Lt[0, 0, [2, 4]] = 5.0           # tie: lowest id wins
    Lt[0, 1, 1] = 3.0
    Lt[0, 2, 5] = 1.0                # bonus row
    a, out, diag = greedy_verify(Lt, np.array([[2, 1]]))
    assert a.tolist() == [2] and out.tolist() == [[2, 1, 5]]
    assert diag["top2_gap"][0, 0] == 0.0
    a, out, _ = greedy_verify(Lt, np.array([[4, 1]]))
    assert a.tolist() == [0] and out.tolist() == [[2, -1, -1]]
    a, out, _ = greedy_verify(Lt, np.array([[2, 9]]))   # out-of-range id is never kept
    assert a.tolist() == [1] and out.tolist() == [[2, 1, -1]]


def test_inverse_cdf_edges_and_zero_weights():
    w = np.array([[0.0, 0.25, 0.0, 0.75], [0.0, 0.0, 1.0, 0.0]])
    tok, lo, hi = inverse_cdf(w, np.array([0.25, 0.999]))
    assert tok.tolist() == [3, 2]
    assert lo.tolist() == [0.25, 0.0] and hi.tolist() == [1.0, 1.0]
    tok, _, _ = inverse_cdf(w, np.array([0.0, 0.0]))
    assert tok.tolist() == [1, 2]          # zero-weight ids are never drawn


def test_invariants_random():
    rng = np.random.default_rng(5)
    B, k, V = 2000, 3, 200
    P = softmax(rng.normal(size=(B, k + 1, V)) * 2)
    Q = softmax(np.log(P[:, :k]) + rng.normal(size=(B, k, V)))
    u_acc, u_res, u_draft = verify_uniforms(3, 1, B, k)
    drafts = sample_drafts(Q, u_draft)
    a, out, diag = stochastic_verify(P, Q, drafts, u_acc, u_res)
    rows = np.arange(B)
    assert np.all((a >= 0) & (a <= k))
    for b in range(B):
        assert np.array_equal(out[b, : a[b]], drafts[b, : a[b]])
        assert np.all(out[b, a[b] + 1:] == -1)
        assert 0 <= out[b, a[b]] < V
    rej = a < k
    assert np.all(out[rows[rej], a[rej]] != drafts[rows[rej], a[rej]])
    r = residual_weights(P[rows[rej], a[rej]], Q[rows[rej], a[rej]])
    S = r.sum(-1)
    assert np.all(S > 0)
    np.testing.assert_allclose((r / S[:, None]).sum(-1), 1.0, atol=1e-12)
    assert np.all(r[P[rows[rej], a[rej]] <= Q[rows[rej], a[rej]]] == 0)
    # rejection implies p(d) < q(d) for the rejected draft
    d_rej = drafts[rows[rej], a[rej]]
    assert np.all(P[rows[rej], a[rej], d_rej] < Q[rows[rej], a[rej], d_rej])
    # bad draft ids are rejected
    bad = drafts.copy()
    bad[:, 0] = V + 3
    a2, _, _ = stochastic_verify(P, Q, bad, u_acc, u_res)
    assert np.all(a2 == 0)


def test_metrics_worked_example():
    with open(os.path.join(HERE, "golden", "acceptance_metrics_worked_example.json")) as f:
        ex = json.load(f)
    k = ex["k"]
    n = 1000
    thresholds = [round(x * n / 100) for x in ex["pos_percent"]]   # requests with a >= d
    a = np.zeros(n, dtype=np.int64)
    for d, t in enumerate(thresholds, start=1):
        a[:t] = d
    m = acceptance_metrics(a, k)
    assert [round(100 * x, 1) for x in m["pos"]] == ex["pos_percent"]
    assert round(m["mean_acceptance_length"], 2) == ex["printed_mean_acceptance_length"]
    assert round(100 * m["acceptance_rate"], 1) == ex["printed_acceptance_rate_percent"]
    assert m["num_draft_tokens"] == n * k and m["num_accepted_tokens"] == int(a.sum())
    assert 1.0 <= m["mean_acceptance_length"] <= k + 1
