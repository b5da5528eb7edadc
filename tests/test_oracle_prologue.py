"""Pins for the prologue oracle (RMSNorm, joint Q/K/V projection, head split): closed forms of
the normalisation, torch's own rms_norm and linear in float64 (library routines), a brute-force
fsum evaluation of the whole prologue on tiny shapes, and a projection whose rows pick out
known channels, so that a swapped head order, a transposed matrix, a missing gain, or eps
outside the square root fails one of them."""

import math

import numpy as np
import torch

from oracle import prologue as P
from workloads import generate as G


def test_rms_norm_closed_forms():
    # h = (3, 4): mean square 12.5
    x = P.rms_norm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(x, [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=0, atol=1e-15)
    # a constant row c: x = c / sqrt(c^2 + eps) * g
    for c, eps in ((2.0, 0.0), (0.5, 1e-2), (-3.0, 1e-6)):
        g = np.array([1.0, -2.0, 0.25])
        x = P.rms_norm(np.full((1, 3), c), g, eps)
        assert np.allclose(x, c / math.sqrt(c * c + eps) * g, rtol=1e-15, atol=0)
    # eps = 0, unit gain: mean(x^2) = 1 and the result does not depend on the row's scale
    rng = np.random.default_rng(0)
    h = rng.standard_normal((4, 37))
    x = P.rms_norm(h, np.ones(37), 0.0)
    assert np.allclose(np.mean(x * x, axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(P.rms_norm(h * 1000.0, np.ones(37), 0.0), x, rtol=1e-13, atol=0)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    for d, eps in ((8, 1e-6), (512, 1e-5), (96, 0.3)):
        h = rng.standard_normal((5, d)) * rng.uniform(0.01, 10)
        g = rng.standard_normal(d)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (d,), torch.from_numpy(g), eps).numpy()
        assert np.allclose(P.rms_norm(h, g, eps), ref, rtol=1e-14, atol=1e-15)


def _bf16(x):
    return G.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_projection_rows_pick_known_channels():
    # row j of W is (j + 1) * e_(j mod d): y_j = (j + 1) x_(j mod d), which fixes the row order
    # Q heads, K heads, V heads and the orientation of W
    Hq, H, D, d, B = 4, 2, 8, 16, 3
    n = (Hq + 2 * H) * D
    W = np.zeros((n, d), dtype=np.float32)
    W[np.arange(n), np.arange(n) % d] = np.arange(1, n + 1)
    rng = np.random.default_rng(2)
    h = _bf16(rng.standard_normal((B, d)))
    g = _bf16(rng.uniform(0.5, 1.5, d))
    eps = 1e-5
    x = P.rms_norm(P.bf16_to_f64(h), P.bf16_to_f64(g), eps)
    q, k, v = P.prologue(h, g, _bf16(W), eps, Hq, H, D)
    assert q.shape == (B, Hq, D) and k.shape == (B, H, D) and v.shape == (B, H, D)
    for b in range(B):
        for hq in range(Hq):
            for c in range(D):
                j = hq * D + c
                assert q[b, hq, c] == (j + 1) * x[b, j % d]
        for hk in range(H):
            for c in range(D):
                j = Hq * D + hk * D + c
                assert k[b, hk, c] == (j + 1) * x[b, j % d]
                j2 = (Hq + H) * D + hk * D + c
                assert v[b, hk, c] == (j2 + 1) * x[b, j2 % d]


def test_prologue_brute_force_fsum():
    Hq, H, D, d, B = 2, 1, 4, 8, 2
    rng = np.random.default_rng(3)
    h = _bf16(rng.standard_normal((B, d)) * 3)
    g = _bf16(rng.standard_normal(d))
    W = _bf16(rng.standard_normal(((Hq + 2 * H) * D, d)))
    eps = 1e-3
    q, k, v = P.prologue(h, g, W, eps, Hq, H, D)
    hf, gf, Wf = P.bf16_to_f64(h), P.bf16_to_f64(g), P.bf16_to_f64(W)
    for b in range(B):
        r = 1.0 / math.sqrt(math.fsum(float(t) * float(t) for t in hf[b]) / d + eps)
        xs = [float(hf[b, i]) * r * float(gf[i]) for i in range(d)]
        y = [math.fsum(float(Wf[j, i]) * xs[i] for i in range(d)) for j in range((Hq + 2 * H) * D)]
        got = np.concatenate([q[b].ravel(), k[b].ravel(), v[b].ravel()])
        assert np.allclose(got, y, rtol=1e-13, atol=1e-14)


def test_prologue_matches_torch_linear():
    Hq, H, D, d, B = 4, 2, 16, 256, 5
    rng = np.random.default_rng(4)
    h = _bf16(rng.standard_normal((B, d)))
    g = _bf16(1 + 0.1 * rng.standard_normal(d))
    W = _bf16(rng.standard_normal(((Hq + 2 * H) * D, d)) / math.sqrt(d))
    q, k, v = P.prologue(h, g, W, 1e-6, Hq, H, D)
    th = torch.from_numpy(P.bf16_to_f64(h))
    x = torch.nn.functional.rms_norm(th, (d,), torch.from_numpy(P.bf16_to_f64(g)), 1e-6)
    y = torch.nn.functional.linear(x, torch.from_numpy(P.bf16_to_f64(W))).numpy()
    assert np.allclose(np.concatenate([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], 1), y,
                       rtol=1e-12, atol=1e-13)
