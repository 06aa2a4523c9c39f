"""Seeded synthetic inputs for the verify step: the five workload configurations,
the vocabulary head, target and drafter hidden states.

This module holds none of the verify method's arithmetic. It is the only code the
CPU oracle and the HIP path share: both receive the same bits from here. Draft
tokens are not made here (they are drawn from the drafter distribution, which
needs the head; the oracle draws them for tests, the library's own drafter call
draws them for the benchmark).

Recipe (numpy PCG64, SeedSequence keyed (config id, stream, step)):
  stream 0  W [V, H]:    N(0, 1) * std, then round-to-nearest-even to bf16
                         (fp32 heads stay fp32). Generated in fixed chunks of 2**22
                         elements, each from its own spawned child sequence, so the
                         result does not depend on the thread count.
  stream 1  target hidden h [B, k+1, H] ~ N(0, 1)
  stream 2  drafter noise e [B, k, H] ~ N(0, 1); drafter hidden
            h'[b, j] = rho_j * h[b, j] + sqrt(1 - rho_j**2) * e[b, j] in fp32,
            then rounded like W. rho_j is the config's correlation at depth j+1.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

_CHUNK = 1 << 22


@dataclass(frozen=True)
class Workload:
    """One verify workload: shapes, dtype, head init std, drafter correlation, temperature."""
    cid: int
    name: str
    H: int
    V: int
    B: int
    k: int
    dtype: str            # "bf16" or "f32"
    w_std: float
    rho: tuple            # correlation per depth 1..k
    T: float
    modes: tuple          # subset of ("greedy", "sample")
    steps: int
    seed: int = 0         # Philox seed of the verify call

    @property
    def M_t(self):
        return self.B * (self.k + 1)

    def M_eff(self, mode):
        return self.M_t + (self.B * self.k if mode == "sample" else 0)


def _const_rho(r, k):
    return tuple([r] * k)


def _decay_rho(base, k):
    return tuple(base ** d for d in range(1, k + 1))


WORKLOADS = {
    1: Workload(1, "tiny_f32_H256_V4096_B4_k3", 256, 4096, 4, 3, "f32", 1.0 / math.sqrt(256),
                _const_rho(0.8, 3), 1.0, ("greedy", "sample"), 1),
    2: Workload(2, "decode_H4096_V151936_B1_k3", 4096, 151936, 1, 3, "bf16", 0.02,
                _const_rho(0.9, 3), 1.0, ("greedy",), 1000),
    3: Workload(3, "batched_sample_H5120_V151936_B32_k3", 5120, 151936, 32, 3, "bf16", 0.02,
                _const_rho(0.85, 3), 0.7, ("sample",), 100),
    4: Workload(4, "chained_depth5_H5120_V151936_B64_k5", 5120, 151936, 64, 5, "bf16", 0.02,
                _decay_rho(0.9, 5), 1.0, ("greedy", "sample"), 100),
    5: Workload(5, "rollout_H7168_V129280_B256_k3", 7168, 129280, 256, 3, "bf16", 0.02,
                _const_rho(0.85, 3), 1.0, ("sample",), 200),
}


def custom(H, V, B, k, dtype="bf16", w_std=None, rho=0.85, T=1.0, cid=100, name=None):
    """A workload of arbitrary shape (tests: ragged tails, edge cases)."""
    if w_std is None:
        w_std = 1.0 / math.sqrt(H) if dtype == "f32" else 0.02
    rho_t = tuple(rho) if isinstance(rho, (tuple, list)) else _const_rho(rho, k)
    return Workload(cid, name or f"custom_H{H}_V{V}_B{B}_k{k}_{dtype}", H, V, B, k, dtype,
                    float(w_std), rho_t, float(T), ("greedy", "sample"), 1)


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def round_to_bf16(x32):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def weights(wl: Workload):
    """The shared head W [V, H]: uint16 bf16 bits, or float32 for f32 workloads."""
    n = wl.V * wl.H
    nchunks = (n + _CHUNK - 1) // _CHUNK
    kids = np.random.SeedSequence((wl.cid, 0, 0)).spawn(nchunks)
    out = np.empty(n, dtype=np.uint16 if wl.dtype == "bf16" else np.float32)
    std = np.float32(wl.w_std)

    def fill(i):
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        x = np.random.Generator(np.random.PCG64(kids[i])).standard_normal(hi - lo, dtype=np.float32)
        x *= std
        out[lo:hi] = round_to_bf16(x) if wl.dtype == "bf16" else x

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunks)))
    return out.reshape(wl.V, wl.H)


def hidden(wl: Workload, step: int):
    """(target [B, k+1, H], drafter [B, k, H]) for one step, in the workload's storage dtype."""
    B, k, H = wl.B, wl.k, wl.H
    h = _rng(wl.cid, 1, step).standard_normal((B, k + 1, H), dtype=np.float32)
    e = _rng(wl.cid, 2, step).standard_normal((B, k, H), dtype=np.float32)
    rho = np.asarray(wl.rho, dtype=np.float32).reshape(1, k, 1)
    mix = np.sqrt(np.float32(1.0) - rho * rho).astype(np.float32)
    hd = (rho * h[:, :k, :] + mix * e).astype(np.float32)
    if wl.dtype == "bf16":
        return round_to_bf16(h), round_to_bf16(hd)
    return h, hd


def fuse_inputs(H, V, B, cid=300, step=0, embed=True):
    """Seeded inputs of the MTP input fusion (bf16 bits unless noted):
    stream 4: embedding table E [V, H] ~ N(0, 1) * 0.02 (skipped when embed=False;
              the benchmark passes the head W in its place);
    stream 5: hidden h [B, H] ~ N(0, 1); stream 6: the two norm weights [H] ~ N(1, 0.1);
    stream 7: W_fc [H, 2H] ~ N(0, 1) * 0.02; stream 8: tokens [B] int32 uniform in [0, V).
    """
    E = round_to_bf16(_rng(cid, 4, 0).standard_normal((V, H), dtype=np.float32) * np.float32(0.02)) if embed else None
    h = round_to_bf16(_rng(cid, 5, step).standard_normal((B, H), dtype=np.float32))
    g = _rng(cid, 6, 0).normal(1.0, 0.1, size=(2, H)).astype(np.float32)
    W_fc = round_to_bf16(_rng(cid, 7, 0).standard_normal((H, 2 * H), dtype=np.float32) * np.float32(0.02))
    tokens = _rng(cid, 8, step).integers(0, V, size=B).astype(np.int32)
    return tokens, E, h, round_to_bf16(g[0]), round_to_bf16(g[1]), W_fc


def loss_rows(V, rows, cid=400, step=0, t_std=3.0, s_noise=1.0, quantum=None):
    """Seeded fp32 logits of the draft-loss workload, one generator per row (so any
    subset of rows of a large call can be rebuilt alone):
    stream 9, key (cid, 9, step, n): teacher row T[n] ~ N(0, 1) * t_std, rounded to a
              multiple of `quantum` when given (many equal logits);
    stream 10, key (cid, 10, step, n): student row S[n] = T[n] + N(0, 1) * s_noise.
    Returns (T, S) of shape [len(rows), V].
    """
    rows = list(rows)
    T = np.empty((len(rows), V), dtype=np.float32)
    S = np.empty((len(rows), V), dtype=np.float32)

    def fill(i):
        n = rows[i]
        t = _rng(cid, 9, step, n).standard_normal(V, dtype=np.float32) * np.float32(t_std)
        if quantum is not None:
            t = (np.round(t / np.float32(quantum)) * np.float32(quantum)).astype(np.float32)
        T[i] = t
        S[i] = t + _rng(cid, 10, step, n).standard_normal(V, dtype=np.float32) * np.float32(s_noise)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(rows))))
    return T, S


def loss_inputs(N, V, cid=400, step=0, **kw):
    """All N rows of the draft-loss workload (loss_rows over 0..N-1)."""
    return loss_rows(V, range(N), cid, step, **kw)
