"""Statistical pins of the oracle end to end (Philox uniforms + decision rule + inverse CDF).

10**6 independent requests at V <= 16 share fixed target rows p_0..p_k and drafter
rows q_0..q_{k-1}; drafts are drawn from q with Philox word 2, the verify step uses
words 0 and 1. Chi-square tests (pre-registered threshold p >= 1e-4, fixed seeds so
the outcome is deterministic) check that:
  * the first emitted token follows p_0 ("It's exact, not approximate");
  * the token at slot j, among requests with a >= j, follows p_j;
  * the accepted-length histogram matches the closed form
    P(a = m) = prod_{i<m} alpha_i * (1 - alpha_m), alpha_i = sum_v min(p_i, q_i),
    which for a drafter whose correlation decays with depth gives acceptance that
    falls with depth ("Faster Rollouts with MTP Speculative Decoding", section
    "Enabling MTP": acceptance decays with depth).
"""
import numpy as np
from scipy import stats

from oracle import sample_drafts, stochastic_verify, verify_uniforms, softmax

PMIN = 1e-4


def _rows(rng, n, V, temp=1.5):
    return softmax(rng.normal(size=(n, V)) * temp)


def _alpha(P, Q):
    return np.minimum(P[: Q.shape[0]], Q).sum(-1)


def _run(P, Q, seed, step, B):
    k, V = Q.shape
    u_acc, u_res, u_draft = verify_uniforms(seed, step, B, k)
    Qb = np.broadcast_to(Q, (B, k, V))
    drafts = sample_drafts(Qb, u_draft)
    Pb = np.broadcast_to(P, (B, k + 1, V))
    a, out, _ = stochastic_verify(Pb, Qb, drafts, u_acc, u_res)
    return a, out, drafts


def _gof(counts, probs):
    exp = probs * counts.sum()
    keep = exp > 0
    return stats.chisquare(counts[keep], exp[keep]).pvalue


def test_chi2_emitted_tokens_follow_target():
    rng = np.random.default_rng(2024)
    V, k, B = 12, 3, 1_000_000
    P = _rows(rng, k + 1, V)
    # drafter rows correlated with the target so acceptance is neither 0 nor 1
    Q = softmax(np.log(P[:k]) * 0.7 + rng.normal(size=(k, V)) * 0.6)
    a, out, drafts = _run(P, Q, seed=11, step=3, B=B)
    assert a.min() >= 0 and a.max() <= k
    for j in range(k + 1):
        sel = a >= j
        counts = np.bincount(out[sel, j], minlength=V)
        assert _gof(counts, P[j]) >= PMIN, j
    alpha = _alpha(P, Q)
    reach = np.concatenate([[1.0], np.cumprod(alpha)])
    hist_p = np.array([reach[m] * (1 - alpha[m]) for m in range(k)] + [reach[k]])
    assert _gof(np.bincount(a, minlength=k + 1), hist_p) >= PMIN
    # drafts themselves follow q (Philox word 2 + inverse CDF)
    for j in range(k):
        assert _gof(np.bincount(drafts[:, j], minlength=V), Q[j]) >= PMIN


def test_per_depth_acceptance_decays_with_drafter_correlation():
    """Drafter rows drift further from the target with depth; pos_d must follow prod alpha."""
    rng = np.random.default_rng(77)
    V, k, B = 16, 5, 400_000
    base = rng.normal(size=(k + 1, V)) * 1.5
    P = softmax(base)
    Q = np.stack([softmax(0.9 ** (j + 1) * base[j] + np.sqrt(1 - 0.81 ** (j + 1)) * rng.normal(size=V) * 1.5)
                  for j in range(k)])
    a, _, _ = _run(P, Q, seed=5, step=0, B=B)
    alpha = _alpha(P, Q)
    expected_pos = np.cumprod(alpha)
    observed_pos = np.array([(a >= d).mean() for d in range(1, k + 1)])
    se = np.sqrt(expected_pos * (1 - expected_pos) / B)
    assert np.all(np.abs(observed_pos - expected_pos) <= 5 * se)
    assert np.all(np.diff(observed_pos) < 0)
