"""Exact pins of the oracle's decision rule, in rational arithmetic.

The oracle's own functions run on numpy object arrays of Fractions. For each slot
the uniforms live on the 24-bit grid the verify step uses, and every decision is
monotone in its uniform, so bisection over the grid counts exactly how many grid
points lead to each outcome. From those counts the test builds the exact law of
what the oracle emits and compares it with what the pages fix:

* single slot: the first emitted token is distributed as p ("It's exact, not
  approximate", "Speculative Decoding and MTP: Why Guessing Is Free");
* a chain of k slots: P(a >= j) = prod_{i<j} sum_v min(p_i, q_i) and, given a >= j,
  the token at slot j is distributed as p_j; with k correct guesses a bonus token
  comes from p_k (k correct drafts yield k + 1 tokens: "Speculative Decoding and MTP:
  Why Guessing Is Free", section "Speculative decoding: draft, then verify");
* a context-dependent target: the first two emitted tokens follow the target's
  autoregressive product law.

The only slack is the 24-bit grid: each decision and each inverse-CDF cell is off
by less than 2**-24 from its real-valued probability.

Planted mistakes (a flipped residual, a bonus drawn from the drafter row) must
break these checks, which shows the checks can fail.
"""
from fractions import Fraction as F
import itertools

import numpy as np
import pytest

import oracle.verify as ov

G = 1 << 24


def rand_dist(rng, V, lo=1, hi=60):
    w = rng.integers(lo, hi, size=V)
    s = int(w.sum())
    return np.array([F(int(x), s) for x in w], dtype=object)


def obj(a):
    return np.array(a, dtype=object)


def first_true(pred, n):
    """Parallel bisection: smallest i in [0, G] with pred(i)[e] True, for monotone predicates."""
    lo = np.zeros(n, dtype=np.int64)
    hi = np.full(n, G, dtype=np.int64)
    while np.any(lo < hi):
        mid = (lo + hi) // 2
        res = pred(mid)
        hi = np.where(res & (lo < hi), mid, hi)
        lo = np.where(~res & (lo < hi), mid + 1, lo)
    return lo


def run_oracle(P, Q, drafts, u_acc, u_res):
    """Batch of n independent requests through oracle.stochastic_verify."""
    return ov.stochastic_verify(P, Q, np.asarray(drafts, dtype=np.int64), u_acc, u_res)


def slot_laws(P, Q, d):
    """Exact grid counts for one request: P [k+1, V], Q [k, V], d [k] (objects).

    A[j]    = number of grid u at slot j that keep d[j] (slots before j kept, u = 0).
    R[m][x] = number of grid u' that give token x at slot m, when slot m is the
              first rejection (m < k) or every draft was kept (m = k, bonus).
    """
    k = len(d)
    V = P.shape[-1]

    def batch(n):
        return (np.broadcast_to(P, (n,) + P.shape).copy(),
                np.broadcast_to(Q, (n,) + Q.shape).copy() if k else np.zeros((n, 0, V), dtype=object),
                np.broadcast_to(np.asarray(d, dtype=np.int64), (n, k)).copy())

    A = np.full(k, G, dtype=np.int64)
    if k:
        Pb, Qb, db = batch(k)

        def rejected(i):
            ua = np.full((k, k), F(0), dtype=object)
            for j in range(k):
                ua[j, j] = F(int(i[j]), G)
            a, _, _ = run_oracle(Pb, Qb, db, ua, np.full((k, k + 1), F(0), dtype=object))
            return a <= np.arange(k)                    # slot j rejected <=> a == j
        A = first_true(rejected, k)

    R = np.zeros((k + 1, V), dtype=np.int64)
    slots = [m for m in range(k + 1) if m == k or A[m] < G]
    pairs = [(m, x) for m in slots for x in range(1, V)]
    if pairs:
        n = len(pairs)
        Pb, Qb, db = batch(n)

        def token_at_least(i):
            ua = np.full((n, k), F(0), dtype=object)
            ur = np.full((n, k + 1), F(0), dtype=object)
            for e, (m, x) in enumerate(pairs):
                if m < k:
                    ua[e, m] = F(G - 1, G)              # the largest grid uniform rejects
                ur[e, m] = F(int(i[e]), G)
            a, out, _ = run_oracle(Pb, Qb, db, ua, ur)
            ms = np.array([m for m, _ in pairs])
            assert np.all(a == ms)
            tok = out[np.arange(n), ms]
            return tok >= np.array([x for _, x in pairs])
        bounds = first_true(token_at_least, n)
        edge = {m: [0] + [None] * (V - 1) + [G] for m in slots}
        for (m, x), bnd in zip(pairs, bounds):
            edge[m][x] = int(bnd)
        for m in slots:
            e = edge[m]
            R[m] = [e[x + 1] - e[x] for x in range(V)]
    else:  # V == 1: the only token takes the whole grid
        for m in slots:
            R[m][0] = G
    return A, R


def outcome_law(P, Q, d):
    """Exact law of (a, emitted tokens) for one request with fixed drafts d."""
    k = len(d)
    A, R = slot_laws(P, Q, d)
    law = {}
    reach = F(1)
    for m in range(k + 1):
        if m < k:
            pm = reach * (1 - F(int(A[m]), G))
        else:
            pm = reach
        if pm:
            for x in range(P.shape[-1]):
                if R[m][x]:
                    seq = tuple(int(t) for t in d[:m]) + (x,)
                    law[seq] = law.get(seq, F(0)) + pm * F(int(R[m][x]), G)
        if m < k:
            reach *= F(int(A[m]), G)
    return law


def draft_mixture(P_rows_fn, Q_rows_fn, k, V):
    """Law of emitted sequences when drafts are drawn from the drafter rows."""
    total = {}
    for d in itertools.product(range(V), repeat=k):
        Qd = Q_rows_fn(d)
        pd = F(1)
        for j in range(k):
            pd *= Qd[j][d[j]]
        if pd == 0:
            continue
        for seq, pr in outcome_law(P_rows_fn(d), Qd, obj(d)).items():
            total[seq] = total.get(seq, F(0)) + pd * pr
    return total


def marginal_first(law, V):
    out = [F(0)] * V
    for seq, pr in law.items():
        out[seq[0]] += pr
    return out


# ------------------------------------------------------------------ single slot

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_single_slot_law_is_target(seed):
    rng = np.random.default_rng(seed)
    V = 5
    p, q = rand_dist(rng, V), rand_dist(rng, V)
    law = draft_mixture(lambda d: np.stack([p, p]), lambda d: np.stack([q]), 1, V)
    first = marginal_first(law, V)
    assert sum(law.values()) == 1
    for x in range(V):
        assert abs(first[x] - p[x]) <= F(3, G), (x, float(first[x]), float(p[x]))


def test_single_slot_residual_sign_is_pinned(monkeypatch):
    """A residual of max(0, q - p) instead of max(0, p - q) must break the law."""
    rng = np.random.default_rng(5)
    V = 5
    p, q = rand_dist(rng, V), rand_dist(rng, V)
    flipped = lambda pp, qq: ov.np.where(qq - pp > 0, qq - pp, (qq - pp) * 0)
    monkeypatch.setattr(ov, "residual_weights", flipped)
    law = draft_mixture(lambda d: np.stack([p, p]), lambda d: np.stack([q]), 1, V)
    first = marginal_first(law, V)
    assert max(abs(first[x] - p[x]) for x in range(V)) > F(1, 1000)


# ------------------------------------------------------------------ chain of slots

def _closed_form_reach(Ps, Qs, j):
    out = F(1)
    for i in range(j):
        out *= sum(min(Ps[i][v], Qs[i][v]) for v in range(len(Ps[i])))
    return out


@pytest.mark.parametrize("seed,k,V", [(10, 2, 4), (11, 3, 3)])
def test_chain_law(seed, k, V):
    rng = np.random.default_rng(seed)
    Ps = np.stack([rand_dist(rng, V) for _ in range(k + 1)])
    Qs = np.stack([rand_dist(rng, V) for _ in range(k)])
    law = draft_mixture(lambda d: Ps, lambda d: Qs, k, V)
    assert sum(law.values()) == 1
    tol = F(4 * (k + 1), G)
    for j in range(k + 1):
        reach = sum(pr for seq, pr in law.items() if len(seq) - 1 >= j)
        assert abs(reach - _closed_form_reach(Ps, Qs, j)) <= tol
        # token at slot j given a >= j is distributed as p_j
        cond = [F(0)] * V
        for seq, pr in law.items():
            if len(seq) - 1 >= j:
                cond[seq[j]] += pr
        for x in range(V):
            assert abs(cond[x] - reach * Ps[j][x]) <= tol, (j, x)
    # k+1 tokens exactly when every draft was kept
    full = sum(pr for seq, pr in law.items() if len(seq) == k + 1)
    assert abs(full - _closed_form_reach(Ps, Qs, k)) <= tol


def test_bonus_row_is_pinned(monkeypatch):
    """Drawing the bonus from the drafter's last row instead of p_k must break the chain law."""
    rng = np.random.default_rng(21)
    k, V = 2, 3
    Ps = np.stack([rand_dist(rng, V) for _ in range(k + 1)])
    Qs = np.stack([rand_dist(rng, V) for _ in range(k)])
    real = ov.stochastic_verify

    def wrong(P, Q, drafts, u_acc, u_res):
        P2 = P.copy()
        P2[:, k, :] = Q[:, k - 1, :]                  # planted: bonus row taken from q_{k-1}
        a, out, diag = real(P2, Q, drafts, u_acc, u_res)
        return a, out, diag
    monkeypatch.setattr(ov, "stochastic_verify", wrong)
    law = draft_mixture(lambda d: Ps, lambda d: Qs, k, V)
    reach = sum(pr for seq, pr in law.items() if len(seq) == k + 1)
    cond = [F(0)] * V
    for seq, pr in law.items():
        if len(seq) == k + 1:
            cond[seq[k]] += pr
    assert max(abs(cond[x] - reach * Ps[k][x]) for x in range(V)) > F(1, 1000)


# -------------------------------------------------------- context-dependent target

def test_two_token_autoregressive_law():
    """Target and drafter are first-order Markov chains over V tokens. The first two
    tokens the speculative loop emits must follow p(x1 | c) p(x2 | x1)."""
    rng = np.random.default_rng(7)
    V, k, c = 3, 2, 1
    Pm = np.stack([rand_dist(rng, V) for _ in range(V)])   # Pm[prev] = p(. | prev)
    Qm = np.stack([rand_dist(rng, V) for _ in range(V)])

    def rows(ctx, d, M, n):
        prev = [ctx] + list(d)
        return np.stack([M[prev[j]] for j in range(n)])

    def call_law(ctx):
        return draft_mixture(lambda d: rows(ctx, d, Pm, k + 1), lambda d: rows(ctx, d, Qm, k), k, V)

    first_call = call_law(c)
    next_first = {x: marginal_first(call_law(x), V) for x in range(V)}
    joint = np.full((V, V), F(0), dtype=object)
    for seq, pr in first_call.items():
        if len(seq) >= 2:
            joint[seq[0], seq[1]] += pr
        else:  # one token emitted: the second comes from the next verify call
            for x2 in range(V):
                joint[seq[0], x2] += pr * next_first[seq[0]][x2]
    tol = F(20, G)
    for x1 in range(V):
        for x2 in range(V):
            assert abs(joint[x1, x2] - Pm[c][x1] * Pm[x1][x2]) <= tol, (x1, x2)
