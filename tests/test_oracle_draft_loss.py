"""Pins of the top-k soft cross-entropy draft-loss oracle against things other than itself.

* top-k selection: brute force over every k-subset of a small integer-valued row (the
  selected set has the largest sum, and among those the lexicographically smallest
  indices: lower index wins a tie), plus a hand-worked row with ties and signed zeros;
* k = 1: the ordinary hard-label cross-entropy with the teacher's argmax as the label
  (scipy's logsumexp);
* k = V: the full soft cross-entropy, which equals the teacher's entropy plus
  KL(teacher || student) (scipy.stats.entropy for both);
* student = teacher: the closed form H(pt) - log P_K, with P_K the teacher mass on K;
* shifting either row by a constant leaves the loss unchanged;
* the gradient agrees with central finite differences of the loss, and each row of it
  sums to zero.
"""
import itertools

import numpy as np
import pytest
from scipy.special import logsumexp, softmax
from scipy.stats import entropy

import oracle
import synth


def test_topk_brute_force_small_integer_rows():
    rng = np.random.default_rng(7)
    for trial in range(40):
        V = int(rng.integers(1, 9))
        k = int(rng.integers(1, V + 1))
        t = rng.integers(-3, 4, size=V).astype(np.float32)      # small integers: many ties, exact sums
        best = None
        for sub in itertools.combinations(range(V), k):          # ascending index tuples, lexicographic order
            val = sum(float(t[i]) for i in sub)
            if best is None or val > best[0]:
                best = (val, sub)
        got = oracle.topk_teacher(t, k)
        assert sorted(got.tolist()) == list(best[1]), (t, k, got, best)
        # and ordered by logit descending, index ascending
        for a, b in zip(got[:-1], got[1:]):
            assert t[a] > t[b] or (t[a] == t[b] and a < b)


def test_topk_hand_worked_ties_and_signed_zero():
    t = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 1.5, -0.0, 0.0], dtype=np.float32)
    assert oracle.topk_teacher(t, 2).tolist() == [1, 2]
    assert oracle.topk_teacher(t, 4).tolist() == [1, 2, 4, 5]
    assert oracle.topk_teacher(t, 7).tolist() == [1, 2, 4, 5, 0, 6, 7]   # -0.0 ties +0.0: lower index first


def test_k1_is_hard_label_cross_entropy():
    T, S = synth.loss_rows(300, range(5), cid=401)
    for n in range(5):
        y = int(np.argmax(T[n]))
        loss, idx, pt, _ = oracle.draft_loss_row(T[n], S[n], 1)
        assert idx.tolist() == [y] and pt.tolist() == [1.0]
        ref = logsumexp(S[n].astype(np.float64)) - float(S[n, y])
        assert abs(loss - ref) <= 1e-12 * max(1.0, abs(ref))


def test_full_vocabulary_is_entropy_plus_kl():
    T, S = synth.loss_rows(257, range(4), cid=402)
    for n in range(4):
        loss, _, _, _ = oracle.draft_loss_row(T[n], S[n], 257)
        p = softmax(T[n].astype(np.float64))
        q = softmax(S[n].astype(np.float64))
        ref = entropy(p) + entropy(p, q)
        assert abs(loss - ref) <= 1e-10 * max(1.0, abs(ref)), (loss, ref)


@pytest.mark.parametrize("k", [1, 3, 64, 200])
def test_student_equal_to_teacher_closed_form(k):
    T, _ = synth.loss_rows(500, range(3), cid=403)
    for n in range(3):
        loss, idx, pt, _ = oracle.draft_loss_row(T[n], T[n], k)
        p = softmax(T[n].astype(np.float64))
        PK = p[idx].sum()
        ref = entropy(p[idx] / PK) - np.log(PK)
        assert abs(loss - ref) <= 1e-10 * max(1.0, abs(ref)), (loss, ref)
        assert loss >= -1e-12


def test_shift_invariance():
    T, S = synth.loss_rows(400, range(3), cid=404)
    base, Kb = oracle.draft_loss(T, S, 50)
    shifted, Ks = oracle.draft_loss(T + np.float32(4.0), S - np.float32(3.0), 50)
    assert np.array_equal(Kb, Ks)
    assert np.allclose(base, shifted, rtol=0, atol=1e-5)   # fp32 shifts round the inputs by <= 2^-21


def test_gradient_matches_finite_differences():
    T, S = synth.loss_rows(60, range(2), cid=405)
    k, scale, h = 7, 0.25, 1e-6
    G = oracle.draft_loss_grad(T, S, k, scale)
    rng = np.random.default_rng(3)
    for n in range(2):
        K = set(oracle.topk_teacher(T[n], k).tolist())
        cols = list(K)[:3] + rng.integers(0, 60, size=4).tolist()
        for v in cols:
            sp = S[n].astype(np.float64).copy()
            sm = sp.copy()
            sp[v] += h
            sm[v] -= h
            lp, _, _, _ = oracle.draft_loss_row(T[n], sp, k)
            lm, _, _, _ = oracle.draft_loss_row(T[n], sm, k)
            fd = scale * (lp - lm) / (2 * h)
            assert abs(G[n, v] - fd) <= 1e-7, (n, v, G[n, v], fd)
        assert abs(G[n].sum()) <= 1e-12


def test_synth_rows_are_independent_of_the_subset():
    T_all, S_all = synth.loss_inputs(6, 100, cid=406)
    T_sub, S_sub = synth.loss_rows(100, [4, 1], cid=406)
    assert np.array_equal(T_sub, T_all[[4, 1]]) and np.array_equal(S_sub, S_all[[4, 1]])
    Tq, _ = synth.loss_rows(100, [0], cid=406, quantum=0.5)
    assert np.all(np.fmod(Tq, 0.5) == 0)
