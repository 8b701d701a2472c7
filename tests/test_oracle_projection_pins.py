"""Pins of the projection oracle (oracle/projection.py) against facts that do
not come from its own code.

Page "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1: Q, K, V =
SiLU of the layer input's projections; the gate sigmoid(.) takes the input
through a projection of its own (its pre-activation is returned unactivated).
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from oracle import projection as P


def silu_tanh(x):
    return x * 0.5 * (1.0 + np.tanh(0.5 * x))


def test_against_a_python_triple_loop():
    """Every output of a small case against sums written out element by
    element in pure Python (math.exp for the feature map)."""
    rng = np.random.default_rng(1)
    T, K, F = 3, 7, 2
    h = rng.standard_normal((T, K))
    W = rng.standard_normal((4 * F, K))
    got = P.project(h, W, F)
    for t in range(T):
        for blk in range(4):
            for f in range(F):
                s = 0.0
                for kk in range(K):
                    s += float(h[t, kk]) * float(W[blk * F + f, kk])
                want = s / (1.0 + math.exp(-s)) if blk < 3 else s
                assert abs(got[blk][t, f] - want) <= 1e-13 * max(1.0, abs(want))


def test_selection_weights_give_silu_of_inputs():
    """Rows of W that are unit vectors pick input columns: q[:, f] =
    SiLU(hidden[:, pi(f)]), and the gate block returns the columns as they are."""
    rng = np.random.default_rng(2)
    T, K, F = 50, 40, 8
    h = rng.standard_normal((T, K)) * 3
    pi = rng.permutation(K)[:4 * F] % K
    W = np.zeros((4 * F, K))
    W[np.arange(4 * F), pi] = 1.0
    q, k, v, xg = P.project(h, W, F)
    for blk, out in enumerate((q, k, v)):
        assert np.abs(out - silu_tanh(h[:, pi[blk * F:(blk + 1) * F]])).max() < 1e-14
    assert np.array_equal(xg, h[:, pi[3 * F:]])


def test_constant_inputs_closed_form():
    """hidden = c everywhere and row n of W constant w_n: P[:, n] = K c w_n."""
    T, K, F = 5, 64, 4
    c = 0.25
    wn = np.linspace(-1, 1, 4 * F)
    W = np.repeat(wn[:, None], K, axis=1)
    q, k, v, xg = P.project(np.full((T, K), c), W, F, featurize=False)
    pre = K * c * wn
    for blk, out in enumerate((q, k, v, xg)):
        assert np.abs(out - pre[None, blk * F:(blk + 1) * F]).max() < 1e-14
    qf, _, _, xgf = P.project(np.full((T, K), c), W, F)
    assert np.abs(qf - silu_tanh(pre[None, :F])).max() < 1e-15
    assert np.array_equal(xgf, xg)


def test_rows_and_bf16_widening():
    """Sampled rows equal the full result's rows; bf16 tensors widen exactly."""
    g = torch.Generator().manual_seed(3)
    T, K, F = 40, 128, 16
    h = torch.randn((T, K), generator=g).to(torch.bfloat16)
    W = torch.randn((4 * F, K), generator=g).to(torch.bfloat16)
    full = P.project(h, W, F)
    rows = [0, 7, 7, 39]
    part = P.project(h, W, F, rows=rows)
    for a, b in zip(full, part):
        assert np.array_equal(a[rows], b)
    ref = h.double().numpy() @ W.double().numpy().T
    assert np.abs(full[3] - ref[:, 3 * F:]).max() < 1e-12


def test_composition_with_the_path_oracle():
    """The path on the projection's pre-activations (SiLU inside the path)
    equals the path on the projection's features (SiLU in the projection):
    the feature map moves, nothing else changes -- gate included."""
    rng = np.random.default_rng(4)
    T, K, H, d = 40, 32, 2, 16
    F = H * d
    h = rng.standard_normal((T, K)) * 0.3
    W = rng.standard_normal((4 * F, K)) * 0.3
    qp, kp, vp, xg = P.project(h, W, F, featurize=False)
    qf, kf, vf, xg2 = P.project(h, W, F, featurize=True)
    assert np.array_equal(xg, xg2)
    shp = (T, H, d)
    a, _, _ = O.forward(qp.reshape(shp), kp.reshape(shp), vp.reshape(shp), xg, gated=True)
    b, _, _ = O.forward(qf.reshape(shp), kf.reshape(shp), vf.reshape(shp), xg, gated=True,
                        featurized=True)
    assert np.abs(a - b).max() <= 1e-12 * np.sqrt(np.mean(a ** 2))


def test_rejects_mismatched_weight():
    with pytest.raises(ValueError):
        P.project(np.zeros((2, 8)), np.zeros((12, 8)), 4)
    with pytest.raises(ValueError):
        P.project(np.zeros((2, 8)), np.zeros((16, 9)), 4)
