"""The seeded input generator: determinism, shapes, bf16 rounding, correlation recipe."""
import numpy as np
import torch

import synth


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.normal(size=100_000) * rng.choice([1e-3, 1, 50], size=100_000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(synth.round_to_bf16(x), ref)


def test_weights_deterministic_and_scaled():
    wl = synth.custom(H=64, V=3000, B=2, k=3)
    w1, w2 = synth.weights(wl), synth.weights(wl)
    assert w1.dtype == np.uint16 and w1.shape == (3000, 64)
    assert np.array_equal(w1, w2)
    vals = synth.bf16_to_f32(w1)
    assert abs(vals.std() - 0.02) < 0.001
    f = synth.weights(synth.custom(H=64, V=100, B=1, k=1, dtype="f32"))
    assert f.dtype == np.float32 and abs(f.std() - 1 / 8) < 0.01


def test_hidden_correlation():
    wl = synth.custom(H=4096, V=16, B=8, k=3, rho=(0.9, 0.81, 0.729))
    h, hd = synth.hidden(wl, step=3)
    assert h.shape == (8, 4, 4096) and hd.shape == (8, 3, 4096)
    hf, hdf = synth.bf16_to_f32(h), synth.bf16_to_f32(hd)
    for j, rho in enumerate(wl.rho):
        c = np.corrcoef(hf[:, j].ravel(), hdf[:, j].ravel())[0, 1]
        assert abs(c - rho) < 0.01
    h2, _ = synth.hidden(wl, step=4)
    assert not np.array_equal(h, h2)


def test_configs_shapes():
    c = synth.WORKLOADS
    assert (c[2].M_t, c[3].M_eff("sample"), c[4].M_t, c[5].M_eff("sample")) == (4, 224, 384, 1792)
    assert c[1].dtype == "f32" and c[3].T == 0.7 and c[4].rho[0] == 0.9
