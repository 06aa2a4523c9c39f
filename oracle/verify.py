"""Plain fp64 oracle of the vocab-side verify step (test infrastructure only).

Shapes and names follow the method's own notation:
  B requests, k drafts per request, H hidden width, V vocabulary size, T temperature.
  Xt [B, k+1, H]  target hidden states at the k+1 verify positions of each request
  Xd [B, k, H]    drafter hidden states, the ones the drafts were sampled from
  W  [V, H]       the one vocabulary head the target and the MTP drafter share
  d  [B, k]       draft tokens; d[b, j] is the guess for slot j
  p_j = softmax(Xt[b, j] . W^T / T)   target distribution at slot j (j = 0..k)
  q_j = softmax(Xd[b, j] . W^T / T)   drafter distribution d[b, j] was drawn from

Index alignment (reading; it is what makes "three correct guesses give four
tokens" hold, "Speculative Decoding and MTP: Why Guessing Is Free", section
"Speculative decoding: draft, then verify"): draft d[b, j] is judged against p_j;
p_k is used only for the bonus token when all k drafts are kept.

Output: accepted_len a[b] in [0, k] and out[b, k+1] = (d[b, 0..a-1], correction or
bonus at slot a, then -1 padding).

The functions of the decision rule use only numpy operations that also work on
object arrays, so the tests can run them on exact rationals.
"""

import numpy as np


# --------------------------------------------------------------------------- numerics

def decode_bf16(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values (bf16 is the top half of fp32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def lm_head_logits(X, W):
    """Logits through the shared vocabulary head: L[..., v] = sum_h X[..., h] * W[v, h].

    One head serves both the verifier and the MTP drafter ("The Tiny Draft Model
    Hidden Inside Qwen", sections "One step deeper than the main model" and "What
    vLLM and SGLang do with the weights"; "Optimize vLLM speculative decoding with
    FastMTP heads", section "Key features": full-vocabulary head, no reduction).
    fp64 inputs, fp64 matmul.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    lead = X.shape[:-1]
    # one matrix product over all rows (a stacked product would re-read W per row block)
    return (X.reshape(-1, X.shape[-1]) @ W.T).reshape(lead + (W.shape[0],))


def softmax(L, T=1.0):
    """Row distribution softmax(L / T) over the last axis, fp64, max-subtracted.

    The verifier computes a distribution of its own at each drafted position ("The
    Tiny Draft Model Hidden Inside Qwen", section "How the draft becomes real
    output"). The temperature T is applied to both target and drafter rows.
    """
    Z = np.asarray(L, dtype=np.float64) / float(T)
    Z = Z - Z.max(axis=-1, keepdims=True)
    E = np.exp(Z)
    return E / E.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------- decision rule

def _first_false(ok, k):
    """Index of the first False along axis 1, or k if every entry is True."""
    ok = np.asarray(ok, dtype=bool)
    B = ok.shape[0]
    if k == 0:
        return np.zeros(B, dtype=np.int64)
    bad = ~ok
    return np.where(bad.any(axis=1), np.argmax(bad, axis=1), k).astype(np.int64)


def _assemble(drafts, a, fill):
    """out[b] = d[b, :a], then fill[b] at slot a, then -1 ("drop the remaining draft")."""
    B, k = drafts.shape
    slot = np.arange(k + 1)[None, :]
    padded = np.concatenate([drafts, np.full((B, 1), -1, dtype=drafts.dtype)], axis=1)
    out = np.where(slot < a[:, None], padded, -1)
    out[np.arange(B), a] = fill
    return out.astype(np.int32)


def greedy_verify(Lt, drafts):
    """Greedy verification against the target argmax of every slot.

    The drafts are kept up to the first one the target disagrees with, so greedy
    speculative decoding emits the plain greedy sequence ("The Tiny Draft Model
    Hidden Inside Qwen", section "How the draft becomes real output"); the drafts
    after the first wrong one are discarded ("Speculative Decoding and MTP: Why
    Guessing Is Free", section "Speculative decoding: draft, then verify").

    Lt [B, k+1, V] target logits; drafts [B, k]. argmax ties go to the lowest id.
    Returns (a [B], out [B, k+1], diag) where diag["argmax"] is [B, k+1] and
    diag["top2_gap"] the gap between the two largest logits of each row.
    """
    Lt = np.asarray(Lt)
    drafts = np.asarray(drafts, dtype=np.int64)
    B, k1, V = Lt.shape
    k = k1 - 1
    g = np.argmax(Lt, axis=-1)                      # first occurrence on ties
    agree = drafts == g[:, :k]                      # out-of-range ids never agree
    a = _first_false(agree, k)
    out = _assemble(drafts, a, g[np.arange(B), a])
    if V >= 2:
        top2 = np.sort(Lt, axis=-1)[..., -2:]
        gap = top2[..., 1] - top2[..., 0]
    else:
        gap = np.full((B, k1), np.inf)
    return a, out, {"argmax": g, "top2_gap": gap}


def residual_weights(p, q):
    """Un-normalised corrected distribution max(0, p - q) (standard speculative sampling)."""
    diff = p - q
    return np.where(diff > 0, diff, diff * 0)


def inverse_cdf(w, u):
    """Inverse-transform draw from non-negative weights w [N, V] with uniforms u [N].

    Token = smallest v whose ascending-id prefix sum C(v) exceeds u * S, S = C(V-1).
    If rounding leaves no such v, the last v with w(v) > 0 is taken.
    Returns (tokens [N], lo [N], hi [N]) with lo/hi the normalised CDF edges
    C(tok-1)/S and C(tok)/S of the chosen token.
    """
    w = np.asarray(w)
    u = np.asarray(u)
    N, V = w.shape
    C = np.cumsum(w, axis=-1)
    S = C[:, -1]
    target = u * S
    above = np.asarray(C > target[:, None], dtype=bool)
    tok = np.argmax(above, axis=-1)
    positive = np.asarray(w > 0, dtype=bool)
    last_pos = V - 1 - np.argmax(positive[:, ::-1], axis=-1)
    tok = np.where(above.any(axis=-1), tok, last_pos)
    rows = np.arange(N)
    hi = C[rows, tok]
    lo = np.where(tok > 0, C[rows, np.maximum(tok - 1, 0)], hi * 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        return tok.astype(np.int64), lo / S, hi / S


def stochastic_verify(P, Q, drafts, u_acc, u_res):
    """Exact stochastic verification of one draft chain per request.

    P [B, k+1, V] target rows p_0..p_k; Q [B, k, V] drafter rows q_0..q_{k-1};
    drafts [B, k]; u_acc [B, k] and u_res [B, k+1] uniforms in [0, 1).

    Steps, in order:
      1. slot j keeps draft d = drafts[b, j] iff u_acc[b, j] * q_j(d) < p_j(d)
         (acceptance with probability min(1, p/q); an id outside [0, V) is rejected);
      2. a = first rejected slot, or k if none;
      3. a < k: the replacement is drawn from max(0, p_a - q_a) with u_res[b, a]
         (if that residual sums to 0 the draw falls back to p_a);
         a = k: the bonus token is drawn from p_k with u_res[b, k];
      4. out = kept drafts, the drawn token, -1 padding.
    The pages require the surviving tokens to be distributed exactly as the target
    alone would produce them ("It's exact, not approximate"; "The Tiny Draft Model
    Hidden Inside Qwen", section "How the draft becomes real output": first
    rejection -> corrected replacement distribution; k correct drafts yield k + 1
    tokens, "Speculative Decoding and MTP: Why Guessing Is Free", section
    "Speculative decoding: draft, then verify"). Works on float64 or exact-rational
    object arrays.

    Returns (a [B], out [B, k+1], diag).
    """
    drafts = np.asarray(drafts, dtype=np.int64)
    B, k = drafts.shape
    V = P.shape[-1]
    rows = np.arange(B)
    valid = (drafts >= 0) & (drafts < V)
    dc = np.clip(drafts, 0, V - 1)
    if k > 0:
        p_d = np.take_along_axis(P[:, :k, :], dc[..., None], axis=-1)[..., 0]
        q_d = np.take_along_axis(Q, dc[..., None], axis=-1)[..., 0]
        keep = valid & np.asarray(u_acc * q_d < p_d, dtype=bool)
    else:
        p_d = q_d = np.zeros((B, 0))
        keep = np.zeros((B, 0), dtype=bool)
    a = _first_false(keep, k)
    Pa = P[rows, a]
    if k > 0:
        Qa = Q[rows, np.minimum(a, k - 1)]
        rejected = (a < k)[:, None]
        w = np.where(rejected, residual_weights(Pa, Qa), Pa)
    else:
        w = Pa
    S = w.sum(axis=-1)
    w = np.where(np.asarray(S > 0, dtype=bool)[:, None], w, Pa)
    u_used = u_res[rows, a]
    tok, lo, hi = inverse_cdf(w, u_used)
    out = _assemble(drafts, a, tok)
    diag = {"p_d": p_d, "q_d": q_d, "u_acc": u_acc, "valid": valid,
            "u_res": u_used, "cdf_lo": lo, "cdf_hi": hi, "token": tok}
    return a, out, diag


def sample_drafts(Q, u_draft):
    """Drafter side: d[b, j] drawn from q_j by inverse transform with u_draft[b, j].

    The MTP head proposes tokens through the shared vocabulary head ("The Tiny
    Draft Model Hidden Inside Qwen", section "What vLLM and SGLang do with the
    weights"). Here all k drafter rows are given up front, so each slot is an
    independent draw from its own row.
    """
    B, k, V = Q.shape
    if k == 0:
        return np.zeros((B, 0), dtype=np.int32)
    tok, _, _ = inverse_cdf(Q.reshape(B * k, V), np.asarray(u_draft).reshape(B * k))
    return tok.reshape(B, k).astype(np.int32)


# ------------------------------------------------------- ragged draft lengths

def greedy_verify_ragged(Lt, drafts, klen):
    """Greedy verification when request b proposes only its first klen[b] <= k drafts.

    Dynamic draft length is named as coming drafter support ("Faster Rollouts with
    MTP Speculative Decoding", section "What's Next"); the pages give no rule for
    it. Reading: a request with k_b drafts is verified exactly as a call with k =
    k_b would verify it (target rows 0..k_b, bonus at slot k_b); its output row is
    then padded with -1 to k + 1 slots. Drafts at slots >= k_b are ignored.
    """
    Lt = np.asarray(Lt)
    drafts = np.asarray(drafts, dtype=np.int64)
    B, k1, _ = Lt.shape
    a = np.zeros(B, dtype=np.int64)
    out = np.full((B, k1), -1, dtype=np.int32)
    for b in range(B):
        kb = int(klen[b])
        ab, ob, _ = greedy_verify(Lt[b:b + 1, :kb + 1], drafts[b:b + 1, :kb])
        a[b] = ab[0]
        out[b, :kb + 1] = ob[0]
    return a, out


def stochastic_verify_ragged(P, Q, drafts, klen, u_acc, u_res):
    """Stochastic verification with per-request draft counts klen[b] <= k.

    Same reading as greedy_verify_ragged: request b runs the exact rule of
    stochastic_verify on its first k_b slots (p_0..p_kb, q_0..q_(kb-1), uniforms
    of slots 0..k_b), so after k_b acceptances the bonus comes from p_kb.
    """
    drafts = np.asarray(drafts, dtype=np.int64)
    B, k = drafts.shape
    a = np.zeros(B, dtype=np.int64)
    out = np.full((B, k + 1), -1, dtype=np.int32)
    for b in range(B):
        kb = int(klen[b])
        ab, ob, _ = stochastic_verify(P[b:b + 1, :kb + 1], Q[b:b + 1, :kb], drafts[b:b + 1, :kb],
                                      u_acc[b:b + 1, :kb], u_res[b:b + 1, :kb + 1])
        a[b] = ab[0]
        out[b, :kb + 1] = ob[0]
    return a, out


# -------------------------------------------------------------- whole verify calls

def verify_greedy_from_hidden(Xt, W, drafts):
    """Greedy verify call from hidden states: logits -> argmax -> longest agreeing prefix."""
    Lt = lm_head_logits(Xt, W)
    a, out, diag = greedy_verify(Lt, drafts)
    return {"a": a, "out": out, "Lt": Lt, **diag}


def verify_sample_from_hidden(Xt, Xd, W, drafts, T, seed, step, b0=0):
    """Stochastic verify call: logits of target and drafter rows through one head,
    softmax at T, Philox uniforms keyed by (seed; slot, request, step), exact rule."""
    from .philox import verify_uniforms
    drafts = np.asarray(drafts)
    B, k = drafts.shape
    Lt = lm_head_logits(Xt, W)
    Ld = lm_head_logits(Xd, W) if k > 0 else np.zeros((B, 0, Lt.shape[-1]))
    P = softmax(Lt, T)
    Q = softmax(Ld, T) if k > 0 else Ld
    u_acc, u_res, _ = verify_uniforms(seed, step, B, k, b0)
    a, out, diag = stochastic_verify(P, Q, drafts, u_acc, u_res)
    return {"a": a, "out": out, "Lt": Lt, "Ld": Ld, "P": P, "Q": Q, **diag}


def verify_greedy_ragged_from_hidden(Xt, W, drafts, klen):
    """Greedy verify call with per-request draft counts (see greedy_verify_ragged)."""
    Lt = lm_head_logits(Xt, W)
    a, out = greedy_verify_ragged(Lt, drafts, klen)
    return {"a": a, "out": out, "Lt": Lt}


def verify_sample_ragged_from_hidden(Xt, Xd, W, drafts, klen, T, seed, step, b0=0):
    """Stochastic verify call with per-request draft counts; uniforms as in
    verify_sample_from_hidden (slot j, request b)."""
    from .philox import verify_uniforms
    drafts = np.asarray(drafts)
    B, k = drafts.shape
    Lt = lm_head_logits(Xt, W)
    Ld = lm_head_logits(Xd, W) if k > 0 else np.zeros((B, 0, Lt.shape[-1]))
    P = softmax(Lt, T)
    Q = softmax(Ld, T) if k > 0 else Ld
    u_acc, u_res, _ = verify_uniforms(seed, step, B, k, b0)
    a, out = stochastic_verify_ragged(P, Q, drafts, klen, u_acc, u_res)
    return {"a": a, "out": out, "Lt": Lt, "Ld": Ld, "P": P, "Q": Q}


def draft_from_hidden(Xd, W, T, seed, step, b0=0):
    """Drafter rows -> q at T -> one draw per slot with Philox word 2."""
    from .philox import verify_uniforms
    B, k, _ = np.shape(Xd)
    Ld = lm_head_logits(Xd, W)
    Q = softmax(Ld, T)
    _, _, u_draft = verify_uniforms(seed, step, B, k, b0)
    return sample_drafts(Q, u_draft), Q
