"""Pins of the oracle's Philox4x32-10 and of the uniforms the verify step draws.

Independent sources: the Random123 known-answer vectors (golden file) and rocRAND's
own source implementation, built host-only with hipcc and fed a grid of counters
and keys. A chi-square test checks the 24-bit uniforms are uniform.
"""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle.philox import philox4x32_10, uniform24, verify_uniforms

HERE = os.path.dirname(os.path.abspath(__file__))


def _hex(xs):
    return np.array([int(x, 16) for x in xs], dtype=np.uint32)


def test_known_answer_vectors():
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        out = philox4x32_10(_hex(v["counter"]), _hex(v["key"]))
        assert out.tolist() == _hex(v["out"]).tolist()


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("philox") / "ref")
    src = os.path.join(HERE, "philox_ref", "rocrand_ten_rounds.cpp")
    subprocess.run([hipcc, "-O1", src, "-o", exe], check=True, capture_output=True)
    return exe


def test_matches_rocrand_source_on_grid(rocrand_ref):
    rng = np.random.default_rng(1234)
    n = 4000
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    # include the counter layout the verify step uses: (slot, request, step lo, step hi)
    ctr[:200, 0] = np.arange(200) % 7
    ctr[:200, 1] = np.arange(200) // 7
    ctr[:200, 2] = 5
    ctr[:200, 3] = 0
    key[:100] = 0
    lines = "\n".join(" ".join("%x" % x for x in list(c) + list(k)) for c, k in zip(ctr, key))
    res = subprocess.run([rocrand_ref], input=lines, capture_output=True, text=True, check=True)
    ref = np.array([[int(x, 16) for x in ln.split()] for ln in res.stdout.strip().splitlines()],
                   dtype=np.uint32)
    ours = philox4x32_10(ctr, key)
    assert ref.shape == ours.shape
    assert np.array_equal(ref, ours)


def test_uniform24_grid():
    w = np.array([0, 0xFF, 0x100, 0x80000000, 0xFFFFFFFF], dtype=np.uint32)
    u = uniform24(w)
    assert u.tolist() == [0.0, 0.0, 2.0 ** -24, 0.5, 1.0 - 2.0 ** -24]
    assert np.all(u < 1.0)
    # every value is exactly representable in fp32 as well
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)


def test_uniforms_are_uniform_chi2():
    B, k = 1 << 16, 3
    u_acc, u_res, u_draft = verify_uniforms(seed=99, step=7, B=B, k=k)
    for u in (u_acc, u_res, u_draft):
        counts = np.bincount((u.ravel() * 64).astype(np.int64), minlength=64)
        assert stats.chisquare(counts).pvalue > 1e-4


def test_verify_uniform_layout():
    """Word 0 / 1 / 2 of Philox(seed; j, b, step) feed acceptance / correction / drafting."""
    seed, step, B, k = 0x123456789ABCDEF0, (1 << 33) + 5, 3, 2
    u_acc, u_res, u_draft = verify_uniforms(seed, step, B, k)
    for b in range(B):
        for j in range(k + 1):
            ctr = np.array([j, b, step & 0xFFFFFFFF, step >> 32], dtype=np.uint32)
            key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
            w = philox4x32_10(ctr, key)
            assert u_res[b, j] == uniform24(w[1])
            if j < k:
                assert u_acc[b, j] == uniform24(w[0])
                assert u_draft[b, j] == uniform24(w[2])
    # request offset b0 shifts the request word only
    a2, r2, d2 = verify_uniforms(seed, step, 2, k, b0=1)
    assert np.array_equal(a2, u_acc[1:]) and np.array_equal(r2, u_res[1:])
