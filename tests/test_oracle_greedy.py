"""Greedy equivalence pin: speculative greedy decoding with the oracle's verify step
returns exactly the tokens of ordinary greedy decoding ("The Tiny Draft Model Hidden
Inside Qwen", section "How the draft becomes real output").

Toy causal LM: state s_t = tanh(A s_{t-1} + E[x_t]), logits = W s_t. The drafter is a
perturbed copy of the model. A perfect drafter keeps every draft (a = k); an
adversarial drafter (target argmax + 1 mod V) keeps none (a = 0).
"""
import numpy as np

from oracle import greedy_verify, lm_head_logits


class ToyLM:
    def __init__(self, rng, V, D):
        self.A = rng.normal(size=(D, D)) / np.sqrt(D)
        self.E = rng.normal(size=(V, D))
        self.W = rng.normal(size=(V, D))

    def states(self, tokens, s0):
        s, out = s0, []
        for x in tokens:
            s = np.tanh(self.A @ s + self.E[x])
            out.append(s)
        return np.array(out), s


def plain_greedy(lm, prompt, n, D):
    s = np.zeros(D)
    _, s = lm.states(prompt, s)
    out = []
    for _ in range(n):
        x = int(np.argmax(lm_head_logits(s[None], lm.W)[0]))
        out.append(x)
        _, s = lm.states([x], s)
    return out


def spec_greedy(lm, draft_fn, prompt, n, k, D):
    s = np.zeros(D)
    _, s = lm.states(prompt, s)
    out, lengths = [], []
    while len(out) < n:
        drafts = draft_fn(s, k)
        # target states at the k+1 verify positions: before each draft token, then after the last
        st, _ = lm.states(drafts, s)
        pos_states = np.concatenate([s[None], st], axis=0)           # [k+1, D]
        Lt = lm_head_logits(pos_states, lm.W)[None]                     # [1, k+1, V]
        a, emitted, _ = greedy_verify(Lt, np.array([drafts]))
        toks = [int(t) for t in emitted[0, : a[0] + 1]]
        assert all(t >= 0 for t in toks) and np.all(emitted[0, a[0] + 1:] == -1)
        lengths.append(int(a[0]))
        out.extend(toks)
        _, s = lm.states(toks, s)
    return out[:n], lengths


def make_drafter(lm, noise, rng, mode):
    def draft(s, k):
        toks = []
        for _ in range(k):
            logits = lm_head_logits(s[None], lm.W)[0]
            if mode == "noisy":
                logits = logits + rng.normal(size=logits.shape) * noise
            x = int(np.argmax(logits))
            if mode == "adversarial":
                x = (x + 1) % logits.shape[0]
            toks.append(x)
            _, s = lm.states([x], s)
        return toks
    return draft


def test_spec_greedy_equals_plain_greedy():
    rng = np.random.default_rng(0)
    V, D, k, n = 24, 12, 3, 256
    for prompt_id in range(100):
        lm = ToyLM(np.random.default_rng(1000 + prompt_id % 10), V, D)
        prompt = list(rng.integers(0, V, size=5))
        ref = plain_greedy(lm, prompt, n, D)
        got, lengths = spec_greedy(lm, make_drafter(lm, 1.0, rng, "noisy"), prompt, n, k, D)
        assert got == ref, prompt_id
        assert 0 < np.mean(lengths) < k      # some but not all drafts kept


def test_perfect_and_adversarial_drafters():
    rng = np.random.default_rng(1)
    V, D, k, n = 24, 12, 4, 64
    lm = ToyLM(rng, V, D)
    prompt = [1, 2, 3]
    ref = plain_greedy(lm, prompt, n, D)
    got, lengths = spec_greedy(lm, make_drafter(lm, 0.0, rng, "perfect"), prompt, n, k, D)
    assert got == ref and set(lengths) == {k}
    got, lengths = spec_greedy(lm, make_drafter(lm, 0.0, rng, "adversarial"), prompt, n, k, D)
    assert got == ref and set(lengths) == {0}
