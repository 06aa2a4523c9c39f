"""Pins of the oracle's per-request draft counts (k_b <= k drafts for request b).

Against things other than the ragged functions themselves:
* k_b = 0: nothing is judged, a = 0, and the emitted token is the inverse-CDF draw
  from p_0 that np.searchsorted gives on the cumulative sum (a library routine);
* k_b = 1 with q_0 = p_0: the draft is always kept (u * q < p for u < 1), and the
  bonus is drawn from p_1 (searchsorted again), not from the last row p_k;
* greedy with drafts equal to the row argmaxes: a = k_b and the bonus is the brute
  force argmax of target row k_b; drafts past k_b never matter, even out of range;
* the exact law of a request with k_b = 2 inside a call with k = 3, enumerated in
  rational arithmetic: P(a >= j) = prod_{i<j} sum_v min(p_i, q_i) for j <= 2, and the
  token after two acceptances follows p_2;
* k_b = k everywhere reproduces the fixed-k rule.
"""
from fractions import Fraction as F
import itertools

import numpy as np
import pytest

import oracle.verify as ov


def _dist(rng, n, V):
    x = rng.random((n, V)) + 0.05
    return x / x.sum(axis=-1, keepdims=True)


def test_kb0_draws_from_p0_with_searchsorted():
    rng = np.random.default_rng(1)
    B, k, V = 64, 3, 11
    P, Q = _dist(rng, B * (k + 1), V).reshape(B, k + 1, V), _dist(rng, B * k, V).reshape(B, k, V)
    drafts = rng.integers(0, V, size=(B, k))
    u_acc, u_res = rng.random((B, k)), rng.random((B, k + 1))
    a, out = ov.stochastic_verify_ragged(P, Q, drafts, np.zeros(B, dtype=int), u_acc, u_res)
    assert np.all(a == 0)
    want = [np.searchsorted(np.cumsum(P[b, 0]), u_res[b, 0] * P[b, 0].sum(), side="right") for b in range(B)]
    assert np.array_equal(out[:, 0], want)
    assert np.all(out[:, 1:] == -1)


def test_kb1_bonus_comes_from_row_kb():
    rng = np.random.default_rng(2)
    B, k, V = 64, 4, 9
    P = _dist(rng, B * (k + 1), V).reshape(B, k + 1, V)
    Q = _dist(rng, B * k, V).reshape(B, k, V)
    Q[:, 0] = P[:, 0]                     # q_0 = p_0: the slot-0 draft is always kept
    drafts = rng.integers(0, V, size=(B, k))
    drafts[:, 1:] = -5                    # slots past k_b are ignored, even out of range
    u_acc, u_res = rng.random((B, k)), rng.random((B, k + 1))
    a, out = ov.stochastic_verify_ragged(P, Q, drafts, np.ones(B, dtype=int), u_acc, u_res)
    assert np.all(a == 1)
    assert np.array_equal(out[:, 0], drafts[:, 0])
    want = [np.searchsorted(np.cumsum(P[b, 1]), u_res[b, 1] * P[b, 1].sum(), side="right") for b in range(B)]
    assert np.array_equal(out[:, 1], want)
    assert np.all(out[:, 2:] == -1)


def test_greedy_ragged_full_agreement():
    rng = np.random.default_rng(3)
    B, k, V = 40, 5, 30
    Lt = rng.normal(size=(B, k + 1, V))
    klen = rng.integers(0, k + 1, size=B)
    drafts = np.full((B, k), -3)
    for b in range(B):
        for j in range(klen[b]):
            drafts[b, j] = max(range(V), key=lambda v: (Lt[b, j, v], -v))
    a, out = ov.greedy_verify_ragged(Lt, drafts, klen)
    assert np.array_equal(a, klen)
    for b in range(B):
        kb = klen[b]
        assert out[b, kb] == max(range(V), key=lambda v: (Lt[b, kb, v], -v))
        assert np.all(out[b, kb + 1:] == -1)
        assert np.array_equal(out[b, :kb], drafts[b, :kb])


def test_kb_equal_k_is_fixed_rule():
    rng = np.random.default_rng(4)
    B, k, V = 16, 3, 12
    P, Q = _dist(rng, B * (k + 1), V).reshape(B, k + 1, V), _dist(rng, B * k, V).reshape(B, k, V)
    drafts = rng.integers(0, V, size=(B, k))
    u_acc, u_res = rng.random((B, k)), rng.random((B, k + 1))
    a1, o1, _ = ov.stochastic_verify(P, Q, drafts, u_acc, u_res)
    a2, o2 = ov.stochastic_verify_ragged(P, Q, drafts, np.full(B, k), u_acc, u_res)
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2)
    g1, go1, _ = ov.greedy_verify(np.log(P), drafts)
    g2, go2 = ov.greedy_verify_ragged(np.log(P), drafts, np.full(B, k))
    assert np.array_equal(g1, g2) and np.array_equal(go1, go2)


def _rat(rng, V):
    w = rng.integers(1, 40, size=V)
    return [F(int(x), int(w.sum())) for x in w]


def test_exact_law_kb2_in_k3():
    """Exact law of the emitted sequence of one request with k_b = 2 of k = 3.

    Uniforms take a 3-point grid {0, 1/3, 2/3} per slot; the oracle's outcome for
    every grid cell and every draft sequence is enumerated in rational arithmetic
    and the law is compared with the closed form of the 2-slot chain. The 3-point
    grid makes acceptance probabilities multiples of 1/3, so p and q are chosen
    with p(d)/q(d) on that grid or above 1, and the residual draw is checked
    through its own cell counts.
    """
    V = 3
    # distributions whose ratios p/q lie in {0, 1/3, 2/3} or >= 1
    p0 = [F(1, 6), F(2, 6), F(3, 6)]
    q0 = [F(3, 6), F(2, 6), F(1, 6)]      # ratios 1/3, 1, 3
    p1 = [F(2, 6), F(2, 6), F(2, 6)]
    q1 = [F(2, 6), F(3, 6), F(1, 6)]      # ratios 1, 2/3, 2
    p2 = [F(1, 2), F(1, 4), F(1, 4)]      # bonus row for k_b = 2
    p3 = [F(0), F(0), F(1)]               # row k = 3: must never be used
    q2 = [F(1, 3)] * 3
    P = np.array([[p0, p1, p2, p3]], dtype=object)
    Q = np.array([[q0, q1, q2]], dtype=object)
    grid = [F(0), F(1, 3), F(2, 3)]
    law = {}
    for d0, d1 in itertools.product(range(V), repeat=2):
        pd = q0[d0] * q1[d1]
        drafts = np.array([[d0, d1, 0]])
        for ua0, ua1 in itertools.product(grid, repeat=2):
            for ur in grid:
                u_acc = np.array([[ua0, ua1, F(0)]], dtype=object)
                # residual / bonus uniforms: same value at every slot (only slot a is used)
                u_res = np.array([[ur, ur, ur, ur]], dtype=object)
                a, out = ov.stochastic_verify_ragged(P, Q, drafts, [2], u_acc, u_res)
                seq = tuple(int(t) for t in out[0] if t >= 0)
                law[seq] = law.get(seq, F(0)) + pd * F(1, 27)
    assert sum(law.values()) == 1
    # closed form of the reach probabilities on this grid: P(keep slot) = sum_d q(d) * P(u * q(d) < p(d))
    keep = lambda p, q: sum(q[d] * F(sum(1 for u in grid if u * q[d] < p[d]), 3) for d in range(V))
    reach1 = keep(p0, q0)
    reach2 = reach1 * keep(p1, q1)
    got_reach2 = sum(pr for seq, pr in law.items() if len(seq) == 3)
    assert got_reach2 == reach2
    # after two acceptances the third token is the bonus from p2 on the 3-point grid:
    # cells u in {0, 1/3, 2/3} pick the tokens whose CDF interval contains u
    bonus = [F(0)] * V
    for seq, pr in law.items():
        if len(seq) == 3:
            bonus[seq[2]] += pr
    cdf = np.cumsum([float(x) for x in p2])
    cells = [int(np.searchsorted(cdf, float(u), side="right")) for u in grid]
    for x in range(V):
        assert bonus[x] == reach2 * F(cells.count(x), 3)
    assert bonus[2] != reach2 * 1      # not the row-k distribution, which puts all mass on token 2
