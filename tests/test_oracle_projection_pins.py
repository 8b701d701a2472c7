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


# ---- the output projection (page "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南",
# FAQ Q5: the attention layer's Q, K, V and O projection matrices) ----


def test_out_projection_against_a_python_triple_loop():
    """Every output of a small case against sums written out in pure Python."""
    rng = np.random.default_rng(11)
    T, F, N = 3, 5, 4
    y = rng.standard_normal((T, F))
    W = rng.standard_normal((N, F))
    got = P.out_project(y, W)
    assert got.shape == (T, N)
    for t in range(T):
        for n in range(N):
            s = 0.0
            for f in range(F):
                s += float(y[t, f]) * float(W[n, f])
            assert abs(got[t, n] - s) <= 1e-13 * max(1.0, abs(s))


def test_out_projection_selection_and_constants():
    """Unit-vector weight rows select (and scale) input features exactly;
    constant inputs times constant rows give F * c * w."""
    rng = np.random.default_rng(12)
    T, F = 6, 8
    y = rng.standard_normal((T, F))
    perm = [3, 0, 7, 7, 1]
    W = np.zeros((len(perm), F))
    for n, f in enumerate(perm):
        W[n, f] = 2.0 if n % 2 else 1.0
    got = P.out_project(y, W)
    for n, f in enumerate(perm):
        assert np.array_equal(got[:, n], y[:, f] * (2.0 if n % 2 else 1.0))
    c = P.out_project(np.full((2, F), 0.5), np.full((3, F), -0.25))
    assert np.array_equal(c, np.full((2, 3), F * 0.5 * -0.25))


def test_out_projection_column_split_sums_to_the_whole():
    """The heads of a layer split over devices: each holds some columns of y
    and the matching columns of W_o; the per-device partial products add up
    to the product over all heads."""
    rng = np.random.default_rng(13)
    T, F, N = 9, 12, 7
    y = rng.standard_normal((T, F))
    W = rng.standard_normal((N, F))
    whole = P.out_project(y, W)
    parts = sum(P.out_project(y[:, a:b], W[:, a:b]) for a, b in ((0, 4), (4, 9), (9, 12)))
    assert np.abs(whole - parts).max() <= 1e-12 * np.abs(whole).max()


def test_out_projection_linearity_rows_and_bf16():
    """Linear in y; sampled rows equal the full rows; bf16 widens exactly."""
    g = torch.Generator().manual_seed(14)
    T, F, N = 20, 64, 24
    y1 = torch.randn((T, F), generator=g).to(torch.bfloat16)
    y2 = torch.randn((T, F), generator=g).to(torch.bfloat16)
    W = torch.randn((N, F), generator=g).to(torch.bfloat16)
    a = P.out_project(y1, W)
    b = P.out_project(y2, W)
    ab = P.out_project(3.0 * y1.double().numpy() + y2.double().numpy(), W)
    assert np.abs(ab - (3.0 * a + b)).max() <= 1e-12 * np.abs(ab).max()
    rows = [0, 19, 5, 5]
    assert np.array_equal(P.out_project(y1, W, rows=rows), a[rows])
    assert np.array_equal(a, y1.double().numpy() @ W.double().numpy().T)


def test_out_projection_rejects_mismatched_weight():
    with pytest.raises(ValueError):
        P.out_project(np.zeros((2, 8)), np.zeros((3, 9)))
    with pytest.raises(ValueError):
        P.out_project(np.zeros(8), np.zeros((3, 8)))
