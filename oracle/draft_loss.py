"""Oracle of the top-k soft cross-entropy draft loss (test infrastructure only).

"Faster Rollouts with MTP Speculative Decoding" (SkyRL docs), sections "Overview" and
"How does it work?": the MTP head is trained against the policy's own next-token
distribution with a soft cross-entropy restricted to the policy's top-k tokens
(k = 256 in the section "Example"); the teacher (the policy) is detached, so only the
head's logits receive a gradient, and the loss is computed per vocabulary shard under
tensor parallelism. The page names the loss and its knob but prints no formula.
Readings taken here (the plainest ones the page supports):

* teacher distribution p = softmax of the teacher logits at temperature 1;
* K = the k tokens with the largest teacher logits; equal logits go to the lower token
  index (so K is unique); -0.0 and +0.0 count as equal;
* soft targets = p restricted to K and renormalized, which is softmax over the k
  selected teacher logits alone (the full teacher normalizer cancels);
* student log-probabilities are normalized over the whole vocabulary:
  log q_v = s_v - logsumexp(s);
* loss of a row = - sum_{j in K} pt_j * log q_j = logsumexp(s) - sum_{j in K} pt_j s_j;
* gradient with respect to the student logits (the teacher gets none):
  dL/ds_v = q_v - pt_v [v in K], scaled by the caller's upstream factor.

Everything in fp64 from the exactly converted fp32 inputs.
"""
import numpy as np


def topk_teacher(t_row, k):
    """Indices of the k largest teacher logits, ordered by (logit desc, index asc)."""
    t = np.asarray(t_row, dtype=np.float64) + 0.0   # -0.0 + 0.0 == +0.0
    order = np.lexsort((np.arange(t.shape[0]), -t))  # last key is the primary one
    return order[:k]


def soft_targets(t_row, idx):
    """Teacher probabilities on the selected tokens, renormalized over them."""
    tk = np.asarray(t_row, dtype=np.float64)[idx]
    e = np.exp(tk - tk.max())
    return e / e.sum()


def logsumexp(s_row):
    s = np.asarray(s_row, dtype=np.float64)
    m = s.max()
    return m + np.log(np.exp(s - m).sum())


def draft_loss_row(t_row, s_row, k):
    """(loss, K, pt, lse) of one row."""
    idx = topk_teacher(t_row, k)
    pt = soft_targets(t_row, idx)
    lse = logsumexp(s_row)
    s = np.asarray(s_row, dtype=np.float64)
    return lse - np.dot(pt, s[idx]), idx, pt, lse


def draft_loss(T, S, k):
    """Per-row losses [N] and the selected indices [N, k] of teacher T and student S [N, V]."""
    T = np.asarray(T)
    S = np.asarray(S)
    N = T.shape[0]
    loss = np.empty(N, dtype=np.float64)
    K = np.empty((N, k), dtype=np.int64)
    for n in range(N):
        loss[n], K[n], _, _ = draft_loss_row(T[n], S[n], k)
    return loss, K


def draft_loss_grad(T, S, k, scale):
    """scale * dL_n/dS[n, v] for every row: scale * (softmax(S[n]) - pt scattered on K)."""
    T = np.asarray(T)
    S = np.asarray(S, dtype=np.float64)
    G = np.empty(S.shape, dtype=np.float64)
    for n in range(S.shape[0]):
        _, idx, pt, lse = draft_loss_row(T[n], S[n], k)
        g = np.exp(S[n] - lse)
        g[idx] -= pt
        G[n] = scale * g
    return G
