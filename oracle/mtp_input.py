"""Oracle of the MTP module's input fusion in front of the drafter (test infrastructure only).

"The Tiny Draft Model Hidden Inside Qwen", section "One step deeper than the main
model": once a token is chosen, the MTP module takes the main model's final hidden
state and that token's embedding, normalizes both, concatenates them and projects the
result back to the hidden width (the checkpoint lists an `mtp.fc` projection and
three normalization weights, and the module reuses the main model's embedding table:
section "What vLLM and SGLang do with the weights"). The formula itself did not
survive on the page. Readings taken here:

* normalization = RMS normalization with a per-channel weight, eps given by the caller:
  n(x) = x / sqrt(mean(x^2) + eps) * g;
* order of the halves: [n(embedding), n(hidden)] (the page's serving-engine passage
  lists the embedding first; its other passage lists the hidden state first);
* `fc` has no bias: y = [n_e(E[tok]), n_h(h)] @ W_fc^T with W_fc [H, 2H];
* a token outside [0, V) contributes a zero embedding (and the GPU path flags it).

Everything in fp64 from the exactly decoded inputs.
"""
import numpy as np


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis, fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def fused_input(tokens, E, h, g_e, g_h, eps):
    """The 2H-wide fc input [n_e(E[tok]), n_h(h)] per row."""
    tokens = np.asarray(tokens, dtype=np.int64)
    E = np.asarray(E, dtype=np.float64)
    V, H = E.shape
    valid = (tokens >= 0) & (tokens < V)
    emb = np.where(valid[:, None], E[np.clip(tokens, 0, V - 1)], 0.0)
    return np.concatenate([rms_norm(emb, g_e, eps), rms_norm(h, g_h, eps)], axis=-1)


def mtp_input_fuse(tokens, E, h, g_e, g_h, W_fc, eps):
    """y [B, H] = fused_input(...) @ W_fc^T, and the fused input itself."""
    x = fused_input(tokens, E, h, g_e, g_h, eps)
    return x @ np.asarray(W_fc, dtype=np.float64).T, x
