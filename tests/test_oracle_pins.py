"""Pins of the CPU oracle against facts that do not come from its own code.

Each pin names the page passage it follows (page title, then section):
  [Tut]  "六十四：MiniMax-01" (LLM tutorial, lesson 64), section 3
  [Arch] "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1

The brute-force reference below evaluates the masked quadratic
(attention-like) form of [Tut] 3 -- sum over i <= t of
(phi(q_t).phi(k_i)) phi(v_i) -- with numpy matmuls and a tanh-based SiLU,
which shares neither formula nor code with the oracle's token recurrence.
"""
import math

import numpy as np
import pytest

from oracle import oracle as O


def silu_tanh(x):
    # x * sigmoid(x) written through tanh: sigmoid(x) = (1 + tanh(x/2)) / 2
    return x * 0.5 * (1.0 + np.tanh(0.5 * x))


def brute_force(q, k, v, S0=None, z0=None, normalized=False):
    """Masked quadratic form, per head: Y = tril(A B^T) C + A S0, and for the
    normalised mode the same over tril(A B^T) 1 + A z0."""
    T, H, d = q.shape
    a, b, c = silu_tanh(q), silu_tanh(k), silu_tanh(v)
    y = np.zeros((T, H, d))
    for h in range(H):
        P = np.tril(a[:, h] @ b[:, h].T)
        num = P @ c[:, h]
        if S0 is not None:
            num = num + a[:, h] @ S0[h]
        if normalized:
            den = P.sum(axis=1)
            if z0 is not None:
                den = den + a[:, h] @ z0[h]
            num = num / den[:, None]
        y[:, h] = num
    return y


def rel(a, b):
    return np.abs(a - b).max() / max(np.sqrt(np.mean(b ** 2)), 1e-300)


@pytest.mark.parametrize("T", [1, 2, 7, 64, 131])
@pytest.mark.parametrize("with_state", [False, True])
def test_recurrence_equals_masked_quadratic_form(T, with_state):
    rng = np.random.default_rng(100 + T)
    H, d = 3, 16
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    S0 = rng.standard_normal((H, d, d)) * 0.1 if with_state else None
    y, S, _ = O.prefill(q, k, v, state_in=None if S0 is None else S0[None])
    ref = brute_force(q, k, v, S0)
    assert rel(y, ref) < 1e-12
    # final state: S0 + phi(K)^T phi(V)  ([Tut] 3, S_T summed in closed form)
    b, c = silu_tanh(k), silu_tanh(v)
    S_ref = np.einsum("thi,thj->hij", b, c) + (S0 if S0 is not None else 0.0)
    assert np.abs(S[0] - S_ref).max() < 1e-11


@pytest.mark.parametrize("T", [1, 5, 96])
def test_normalized_equals_masked_quadratic_form(T):
    rng = np.random.default_rng(7 + T)
    H, d = 2, 16
    # positive-mean pre-activations keep phi(q).z away from zero
    q, k, v = (2.0 + 0.5 * rng.standard_normal((T, H, d)) for _ in range(3))
    S0 = np.abs(rng.standard_normal((H, d, d)))
    z0 = np.abs(rng.standard_normal((H, d))) + 1.0
    y, S, z = O.prefill(q, k, v, state_in=S0[None], z_in=z0[None], normalized=True)
    ref = brute_force(q, k, v, S0, z0, normalized=True)
    assert rel(y, ref) < 1e-12
    assert np.abs(z[0] - (z0 + silu_tanh(k).sum(axis=0))).max() < 1e-11


@pytest.mark.parametrize("c", [-1.5, 0.25, 1.0, 3.0])
def test_closed_form_constant_inputs(c):
    """All pre-activations equal c, s = SiLU(c): S_t = t s^2 (every entry),
    y_t[j] = d t s^3; normalised y_t = s; gated output = Y/sqrt(Y^2+eps) w sig(x)."""
    T, H, d = 40, 2, 8
    s = c / (1.0 + math.exp(-c))
    q = np.full((T, H, d), c)
    y, S, _ = O.prefill(q, q, q)
    t = np.arange(1, T + 1, dtype=np.float64)
    expect = (d * t * s ** 3)[:, None, None] * np.ones((1, H, d))
    assert np.abs(y - expect).max() <= 1e-13 * np.abs(expect).max()
    assert np.abs(S - T * s * s).max() <= 1e-13 * T * s * s
    yn, _, _ = O.prefill(q, q, q, normalized=True)
    assert np.abs(yn - s).max() <= 1e-13 * abs(s)
    # gate: Y is constant over the token's features, so mean(Y^2) = Y^2
    x = np.full((T, H * d), 0.7)
    w = np.linspace(0.5, 1.5, H * d)
    eps = 1e-6
    out = O.gate(y.reshape(T, H * d), x, w, 0, eps)
    Y = d * t * s ** 3
    sig = 1.0 / (1.0 + math.exp(-0.7))
    expect_g = (Y / np.sqrt(Y * Y + eps))[:, None] * w[None, :] * sig
    assert np.abs(out - expect_g).max() < 1e-14


def test_single_token():
    """T = 1: y = (phi(q).phi(k)) phi(v); normalised: y = phi(v)."""
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 4, 32)) for _ in range(3))
    y, _, _ = O.prefill(q, k, v)
    a, b, cc = silu_tanh(q[0]), silu_tanh(k[0]), silu_tanh(v[0])
    expect = (a * b).sum(axis=1)[:, None] * cc
    assert np.abs(y[0] - expect).max() < 1e-14
    yn, _, _ = O.prefill(q, k, v, normalized=True)
    assert np.abs(yn[0] - cc).max() < 1e-13


def test_last_row_is_noncausal_product():
    """At the last token the causal mask covers every key, so y_T equals the
    non-causal Q (K^T V) of [Arch] 2.1 for that row."""
    rng = np.random.default_rng(5)
    T, H, d = 50, 2, 16
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    y, _, _ = O.prefill(q, k, v)
    a, b, c = silu_tanh(q), silu_tanh(k), silu_tanh(v)
    for h in range(H):
        KV = b[:, h].T @ c[:, h]
        assert np.abs(y[-1, h] - a[-1, h] @ KV).max() < 1e-12


@pytest.mark.parametrize("normalized", [False, True])
def test_state_chaining(normalized):
    """prefill(T1 || T2) == prefill(T2 | state_out(prefill(T1)))."""
    rng = np.random.default_rng(11)
    T1, T2, H, d = 45, 38, 2, 16
    sh = 1.5 if normalized else 0.0
    q, k, v = (sh + rng.standard_normal((T1 + T2, H, d)) for _ in range(3))
    y, S, z = O.prefill(q, k, v, normalized=normalized)
    y1, S1, z1 = O.prefill(q[:T1], k[:T1], v[:T1], normalized=normalized)
    y2, S2, z2 = O.prefill(q[T1:], k[T1:], v[T1:], state_in=S1, z_in=z1, normalized=normalized)
    assert rel(np.concatenate([y1, y2]), y) < 1e-12
    assert np.abs(S2 - S).max() < 1e-11
    if normalized:
        assert np.abs(z2 - z).max() < 1e-11


@pytest.mark.parametrize("normalized", [False, True])
def test_decode_steps_equal_prefill(normalized):
    rng = np.random.default_rng(13)
    T, N, H, d = 12, 3, 2, 16
    sh = 1.5 if normalized else 0.0
    q, k, v = (sh + rng.standard_normal((N, T, H, d)) for _ in range(3))
    S0 = np.abs(rng.standard_normal((N, H, d, d))) * 0.1
    z0 = np.abs(rng.standard_normal((N, H, d))) + 0.5
    S, z = S0.copy(), z0.copy()
    ys = []
    for t in range(T):
        yt, S, z = O.decode_step(q[:, t], k[:, t], v[:, t], S, z, normalized)
        ys.append(yt)
    ys = np.stack(ys, axis=1)  # [N, T, H, d]
    for n in range(N):
        y, Sp, zp = O.prefill(q[n], k[n], v[n], state_in=S0[n:n + 1], z_in=z0[n:n + 1],
                              normalized=normalized)
        assert rel(ys[n], y) < 1e-12
        assert np.abs(S[n] - Sp[0]).max() < 1e-11


def test_varlen_equals_per_sequence():
    rng = np.random.default_rng(17)
    lengths = [5, 1, 0, 33, 64, 2]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    H, d = 2, 16
    q, k, v = (rng.standard_normal((cu[-1], H, d)) for _ in range(3))
    S0 = rng.standard_normal((len(lengths), H, d, d)) * 0.1
    y, S, _ = O.prefill(q, k, v, cu_seqlens=cu, state_in=S0)
    for s, L in enumerate(lengths):
        a, b = cu[s], cu[s + 1]
        ys, Ss, _ = O.prefill(q[a:b], k[a:b], v[a:b], state_in=S0[s:s + 1])
        if L:
            assert rel(y[a:b], ys) < 1e-13
            assert rel(y[a:b], brute_force(q[a:b], k[a:b], v[a:b], S0[s])) < 1e-12
        assert np.abs(S[s] - Ss[0]).max() < 1e-12


def test_sampled_outputs_match_full():
    rng = np.random.default_rng(19)
    T, H, d = 300, 2, 16
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    y, _, _ = O.prefill(q, k, v)
    idx = np.array([0, 0, 17, 150, 299])
    ys, _, _ = O.prefill(q, k, v, sample_idx=idx)
    assert np.array_equal(ys, y[idx])


@pytest.mark.parametrize("B", [32, 64, 128, 256])
def test_block_size_invariance(B):
    """The blocked form (quadratic within a block, state across blocks) is a
    reassociation of the same sum: fp64 agrees to rounding, fp32 to ~1e-6."""
    rng = np.random.default_rng(23)
    T, H, d = 700, 2, 64
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    y, S, _ = O.prefill(q, k, v)
    yb, Sb, _ = O.prefill_blocked(q, k, v, B)
    assert rel(yb, y) < 1e-12 and rel(Sb, S) < 1e-12
    yf, Sf, _ = O.prefill_blocked(q, k, v, B, fp32=True)
    assert rel(yf, y) < 1e-5 and rel(Sf, S) < 1e-5
    ynb, _, _ = O.prefill_blocked(q + 2, k + 2, v, B, normalized=True)
    yn, _, _ = O.prefill(q + 2, k + 2, v, normalized=True)
    assert rel(ynb, yn) < 1e-12


def test_gate_invariants():
    """[Arch] 2.1 output gate.  Dividing out w*sigmoid(x) leaves y*r whose
    mean square over the norm group is m/(m+eps), m = mean(y^2); permuting
    heads consistently in y, x, w permutes the output; x = 0 gives exactly
    half of the normalised y."""
    rng = np.random.default_rng(29)
    T, H, d = 20, 4, 16
    F = H * d
    y = rng.standard_normal((T, F)) * rng.uniform(0.01, 10, size=(T, 1))
    x = rng.standard_normal((T, F))
    w = rng.uniform(0.5, 2.0, size=F)
    eps = 1e-3
    out = O.gate(y, x, w, 0, eps)
    sig = 0.5 * (1.0 + np.tanh(0.5 * x))
    yr = out / (w * sig)
    m = np.mean(y * y, axis=1)
    assert np.abs(np.mean(yr * yr, axis=1) - m / (m + eps)).max() < 1e-12
    perm = rng.permutation(H)
    cols = (perm[:, None] * d + np.arange(d)[None, :]).reshape(-1)
    outp = O.gate(y[:, cols], x[:, cols], w[cols], 0, eps)
    assert np.abs(outp - out[:, cols]).max() < 1e-14
    # per-head groups: each group of d features is normalised on its own
    outg = O.gate(y, x, w, d, eps)
    yg = (outg / (w * sig)).reshape(T, H, d)
    mg = np.mean(y.reshape(T, H, d) ** 2, axis=2)
    assert np.abs(np.mean(yg * yg, axis=2) - mg / (mg + eps)).max() < 1e-12
    out0 = O.gate(y, np.zeros_like(x), None, 0, eps)
    r = 1.0 / np.sqrt(m + eps)
    assert np.abs(out0 - 0.5 * y * r[:, None]).max() < 1e-13 * np.abs(y * r[:, None]).max()
