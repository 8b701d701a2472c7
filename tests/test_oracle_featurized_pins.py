"""Pins of the oracle's features-given mode: q, k and v arrive as feature
vectors phi(.) already -- the feature map applied where they were produced,
e.g. in the epilogue of the projection that computes them ([Arch]
"MiniMax-Text-01 405B MoE模型架构与训练策略解析" 2.1 writes Q, K, V = SiLU(X W))
-- and the oracle uses them as given.

Pinned against: the oracle's default mode fed the pre-activations, with the
features formed here by scipy's logistic function (so the mode must drop the
feature map on all three inputs and change nothing else); a masked quadratic
form with numpy matmuls; and one-token closed forms.
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle as O


def rel(a, b):
    return np.abs(a - b).max() / max(np.sqrt(np.mean(b ** 2)), 1e-300)


def draw(T, H=2, d=16, seed=0, scale=1.0):
    r = np.random.default_rng(seed)
    return [r.standard_normal((T, H, d)) * scale for _ in range(3)]


def phi(x):
    return x * expit(x)


@pytest.mark.parametrize("normalized", [False, True])
def test_features_given_equals_default_mode_on_their_preimages(normalized):
    q, k, v = draw(97, seed=1)
    cu = [0, 40, 40, 97]
    S0 = np.random.default_rng(2).standard_normal((3, 2, 16, 16)) * 0.1
    z0 = np.abs(np.random.default_rng(3).standard_normal((3, 2, 16))) + 1.0
    y0, S_0, z_0 = O.prefill(q, k, v, cu, S0, z0, normalized=normalized)
    y1, S_1, z_1 = O.prefill(phi(q), phi(k), phi(v), cu, S0, z0, normalized=normalized,
                             featurized=True)
    # the two sides form phi with different fp64 logistic routines (last-bit
    # differences), which the normalised mode's division can amplify
    assert rel(y1, y0) < 1e-10 and rel(S_1, S_0) < 1e-12 and rel(z_1, z_0) < 1e-12


def test_features_given_leaves_the_gate_alone():
    q, k, v = draw(33, seed=4)
    x = np.random.default_rng(5).standard_normal((33, 2 * 16))
    a, _, _ = O.forward(q, k, v, x=x, gated=True)
    b, _, _ = O.forward(phi(q), phi(k), phi(v), x=x, gated=True, featurized=True)
    assert rel(b, a) < 1e-12


def test_features_given_decode_and_blocked_forms():
    q, k, v = draw(50, seed=6)
    y, S, _ = O.prefill(q, k, v, featurized=True)
    for block in (1, 7, 32):
        yb, Sb, _ = O.prefill_blocked(q, k, v, block, featurized=True)
        assert rel(yb, y) < 1e-12 and rel(Sb, S) < 1e-12
    # the decode step on its own state matches the prefill token by token
    Sd = np.zeros((1, 2, 16, 16))
    for t in range(50):
        yd, Sd, _ = O.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], Sd, featurized=True)
        assert rel(yd[0], y[t]) < 1e-12


def test_features_given_masked_quadratic_form():
    q, k, v = draw(64, H=3, d=8, seed=7)
    y, _, _ = O.prefill(q, k, v, featurized=True)
    for h in range(3):
        ref = np.tril(q[:, h] @ k[:, h].T) @ v[:, h]
        assert rel(y[:, h], ref) < 1e-12


def test_features_given_one_token_closed_forms():
    q, k, v = draw(1, H=1, d=8, seed=8)
    y, S, _ = O.prefill(q, k, v, featurized=True)
    # y = q^T (k v^T) = (q . k) v ;  S = k v^T
    np.testing.assert_allclose(y[0, 0], np.dot(q[0, 0], k[0, 0]) * v[0, 0], rtol=1e-13)
    np.testing.assert_allclose(S[0, 0], np.outer(k[0, 0], v[0, 0]), rtol=1e-13)
    # normalised: (q . k) v / (q . k) = v
    yn, _, _ = O.prefill(q, k, v, normalized=True, featurized=True)
    np.testing.assert_allclose(yn[0, 0], v[0, 0], rtol=1e-12)
