"""Philox4x32-10 counter-based generator and the uniforms the verify step draws.

Test infrastructure only (see the package docstring).

Philox4x32-10 is the published generator of Salmon, Moraes, Dror & Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11): a 4-word counter and a
2-word key go through ten rounds. Each round multiplies counter words 0 and 2 by
two fixed odd multipliers, keeps the high and low halves of both 64-bit products,
and mixes the high halves with the other two counter words and the key. The key
is bumped by two Weyl constants between rounds.

The pages do not say how the verifier draws its random numbers. The reading used
throughout (both sides implement it independently):

* key     = (low 32 bits of seed, high 32 bits of seed)
* counter = (slot j, request b, low 32 bits of step, high 32 bits of step)
* output word 0 -> uniform for the acceptance test at slot j
* output word 1 -> uniform for the correction / bonus draw made at slot j
* output word 2 -> uniform the drafter uses to sample the draft for slot j
* uniform(x) = (x >> 8) * 2**-24, a 24-bit grid in [0, 1), exact in fp32/fp64.
"""

import numpy as np

# Round multipliers and Weyl key increments from the Philox4x32 definition.
_MUL0 = np.uint64(0xD2511F53)
_MUL1 = np.uint64(0xCD9E8D57)
_WEYL0 = np.uint64(0x9E3779B9)
_WEYL1 = np.uint64(0xBB67AE85)
_LO32 = np.uint64(0xFFFFFFFF)
_SHIFT32 = np.uint64(32)


def philox4x32_10(counter, key):
    """Ten Philox4x32 rounds. counter: uint32 [..., 4]; key: uint32 [..., 2].

    Returns uint32 [..., 4]. Broadcasting follows numpy rules over the leading
    axes. Arithmetic is done in uint64 so each 32x32-bit product is exact.
    """
    counter = np.asarray(counter, dtype=np.uint32).astype(np.uint64)
    key = np.asarray(key, dtype=np.uint32).astype(np.uint64)
    c0, c1, c2, c3 = (counter[..., i] for i in range(4))
    k0, k1 = key[..., 0], key[..., 1]
    for rnd in range(10):
        if rnd > 0:  # key schedule: bump before every round but the first
            k0 = (k0 + _WEYL0) & _LO32
            k1 = (k1 + _WEYL1) & _LO32
        prod0 = c0 * _MUL0
        prod1 = c2 * _MUL1
        hi0, lo0 = prod0 >> _SHIFT32, prod0 & _LO32
        hi1, lo1 = prod1 >> _SHIFT32, prod1 & _LO32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    out = np.stack(np.broadcast_arrays(c0, c1, c2, c3), axis=-1)
    return out.astype(np.uint32)


def uniform24(words):
    """Map uint32 words to the 24-bit grid in [0, 1): (x >> 8) * 2**-24 (fp64)."""
    w = np.asarray(words, dtype=np.uint32)
    return (w >> np.uint32(8)).astype(np.float64) * (2.0 ** -24)


def _key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)


def _counters(B, k, step, b0=0):
    """Counter grid [B, k, 4]: (j, b0 + b, step lo, step hi)."""
    step = int(step) & 0xFFFFFFFFFFFFFFFF
    ctr = np.zeros((B, k, 4), dtype=np.uint32)
    ctr[..., 0] = np.arange(k, dtype=np.uint32)[None, :]
    ctr[..., 1] = (np.arange(B, dtype=np.uint64) + np.uint64(b0)).astype(np.uint32)[:, None]
    ctr[..., 2] = step & 0xFFFFFFFF
    ctr[..., 3] = step >> 32
    return ctr


def verify_uniforms(seed, step, B, k, b0=0):
    """All uniforms one verify call may use, for requests b0..b0+B-1.

    Returns (u_acc [B, k], u_res [B, k+1], u_draft [B, k]):
      u_acc[b, j]   = uniform(word 0 of Philox(seed; j, b, step))
      u_res[b, j]   = uniform(word 1 of Philox(seed; j, b, step))   (j = 0..k)
      u_draft[b, j] = uniform(word 2 of Philox(seed; j, b, step))
    """
    words = philox4x32_10(_counters(B, k + 1, step, b0), _key(seed)[None, None, :])
    u = uniform24(words)
    return u[:, :k, 0], u[:, :, 1], u[:, :k, 2]
