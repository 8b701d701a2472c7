"""Pins of the softmax-layer oracle against facts that do not come from its
own code.

Each pin names the page passage it follows (page title, then section):
  [Tut]      "六十四：MiniMax-01" (LLM tutorial, lesson 64), sections 2-3:
             softmax(Q K^T / sqrt(d)) V
  [Arch]     "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.2:
             rotary embedding on half the dimensions, base 10,000; section
             4.1: base 5M and 10M
  [Overview] "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南",
             section 2.1.3: packed variable-length sequences

Independent references used here: closed forms (zero keys give the running
mean of the values; a two-dimensional rotation gives sin of the position
difference times the frequency; a single key gives its value; a dominant
score gives the hard maximum), and torch's CPU attention routine in fp64
(``_scaled_dot_product_flash_attention_for_cpu``, which also returns the
log-sum-exp) applied to inputs rotated by complex multiplication in numpy.
"""
import math

import numpy as np
import pytest
import torch

from oracle import softmax as SO


def rng(seed):
    return np.random.default_rng(seed)


def library_attention(q, k, v, cu, scale):
    """torch's fp64 CPU causal attention per sequence; k, v repeated over the
    query heads of their group.  Returns (out [T, H, d], lse [T, H])."""
    T, H, d = q.shape
    G = H // k.shape[1]
    out = np.zeros((T, H, d))
    lse = np.zeros((T, H))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        qt = torch.from_numpy(q[a:b]).permute(1, 0, 2).unsqueeze(0)
        kt = torch.from_numpy(np.repeat(k[a:b], G, axis=1)).permute(1, 0, 2).unsqueeze(0)
        vt = torch.from_numpy(np.repeat(v[a:b], G, axis=1)).permute(1, 0, 2).unsqueeze(0)
        o, l = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
            qt.contiguous(), kt.contiguous(), vt.contiguous(), 0.0, True, scale=scale)[:2]
        out[a:b] = o[0].permute(1, 0, 2).numpy()
        lse[a:b] = l[0].permute(1, 0).numpy()
    return out, lse


def rotate_complex(x, cu, rot, base):
    """[Arch] 2.2 rotation written as complex multiplication: the pair
    (j, j + rot/2) is the complex number x_j + i x_{j+rot/2}, multiplied by
    exp(i p base^(-2j/rot)) at position p (counted from each sequence start)."""
    out = x.copy()
    if rot == 0:
        return out
    h = rot // 2
    freq = np.exp(-np.log(base) * (2.0 * np.arange(h) / rot))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        pos = np.arange(b - a, dtype=np.float64)
        z = x[a:b, :, :h] + 1j * x[a:b, :, h:rot]
        z = z * np.exp(1j * np.outer(pos, freq))[:, None, :]
        out[a:b, :, :h] = z.real
        out[a:b, :, h:rot] = z.imag
    return out


def test_zero_keys_give_the_running_mean_of_values():
    # [Tut] 2-3 with every score 0: softmax is uniform over keys u <= t of
    # the sequence, so out_t = mean(v_start .. v_t) and lse = log(count).
    r = rng(1)
    cu = np.array([0, 5, 5, 12, 20])
    T, H, Hkv, d = 20, 4, 2, 16
    q = r.standard_normal((T, H, d))
    k = np.zeros((T, Hkv, d))
    v = r.standard_normal((T, Hkv, d))
    out, lse = SO.attention(q, k, v, cu, rotary_dim=8, rope_base=10000.0)
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            n = t - cu[s] + 1
            mean = v[cu[s]:t + 1].mean(axis=0)
            for h in range(H):
                np.testing.assert_allclose(out[t, h], mean[h // 2], rtol=0, atol=1e-13)
                assert abs(lse[t, h] - math.log(n)) < 1e-13


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_without_rotation_matches_library_attention(H, Hkv):
    # [Tut] 3, causal, scale 1/sqrt(d), packed sequences ([Overview] 2.1.3)
    r = rng(2 + H + Hkv)
    cu = np.array([0, 13, 14, 37])
    T, d = 37, 32
    q, k, v = (r.standard_normal((T, n, d)) for n in (H, Hkv, Hkv))
    out, lse = SO.attention(q, k, v, cu, rotary_dim=0)
    ref, lref = library_attention(q, k, v, cu, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("rot,base", [(16, 10000.0), (32, 5e6), (64, 1e7), (32, 10000.0)])
def test_rotation_matches_complex_multiplication(rot, base):
    # [Arch] 2.2 / 4.1: rotated q and k, then [Tut] 3 attention; the rotation
    # is applied here by complex multiplication and the attention by the
    # library routine.  d = 32 with rot = 16 is "half the dimensions".
    r = rng(int(rot + base) % 1000)
    cu = np.array([0, 40, 41, 90])
    T, H, Hkv, d = 90, 2, 1, (128 if rot == 64 else 32)
    q, k, v = (r.standard_normal((T, n, d)) for n in (H, Hkv, Hkv))
    out, lse = SO.attention(q, k, v, cu, rotary_dim=rot, rope_base=base, scale=0.3)
    ref, lref = library_attention(rotate_complex(q, cu, rot, base), rotate_complex(k, cu, rot, base),
                                  v, cu, 0.3)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lref, rtol=0, atol=1e-11)


def two_key_case(d, rot, base, m, jq, jk, alpha, scale):
    """One sequence of m + 1 tokens: key 0 is the unit vector e_jk, every other
    key is zero; query m is alpha * e_jq; value 0 is e_0, the others zero.
    Returns out[m][0] = weight of key 0."""
    T = m + 1
    q = np.zeros((T, 1, d))
    q[m, 0, jq] = alpha
    k = np.zeros((T, 1, d))
    k[0, 0, jk] = 1.0
    v = np.zeros((T, 1, d))
    v[0, 0, 0] = 1.0
    out, _ = SO.attention(q, k, v, None, rotary_dim=rot, rope_base=base, scale=scale,
                          rows=[m], heads=[0])
    return out[0, 0]


@pytest.mark.parametrize("d,rot,base,m,j", [
    (4, 4, 10000.0, 1, 0),       # theta_0 = 1
    (4, 4, 10000.0, 100, 1),     # theta_1 = 10000^(-1/2) = 0.01, angle 1
    (8, 4, 10000.0, 100, 1),     # half of d = 8
    (128, 64, 1e7, 5000, 31),    # the long-context base, last rotated pair
])
def test_rotation_closed_form(d, rot, base, m, j):
    # [Arch] 2.2: q = alpha e_j at position m, key e_{j+rot/2} at position 0.
    # Rotating the pair (j, j+rot/2) by m*theta_j and 0 gives
    # q' . k' = alpha * sin(m * theta_j), theta_j = base^(-2j/rot); the other
    # m keys score 0, so the weight of key 0 is e^a / (e^a + m).
    alpha, scale = 3.0, 0.7
    theta = base ** (-2.0 * j / rot)
    a = scale * alpha * math.sin(m * theta)
    w = two_key_case(d, rot, base, m, j, j + rot // 2, alpha, scale)
    assert abs(w - math.exp(a) / (math.exp(a) + m)) < 1e-12


def test_dimensions_past_the_rotated_half_are_not_rotated():
    # [Arch] 2.2: only half of the dimensions carry the rotation.  With all
    # of q and k in the unrotated half the scores do not depend on positions:
    # q = alpha e_5, key 0 = e_5 (d = 8, rot = 4): a = scale * alpha.
    alpha, scale, m = 2.0, 0.5, 37
    w = two_key_case(8, 4, 10000.0, m, 5, 5, alpha, scale)
    a = scale * alpha
    assert abs(w - math.exp(a) / (math.exp(a) + m)) < 1e-12


def test_single_token_sequences_return_their_value():
    # one key: softmax weight 1, lse = its score; position 0 rotates by 0.
    r = rng(5)
    T, H, d = 9, 2, 16
    cu = np.arange(T + 1)
    q, k, v = (r.standard_normal((T, H, d)) for _ in range(3))
    out, lse = SO.attention(q, k, v, cu, rotary_dim=8, rope_base=10000.0, scale=0.25)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.25 * np.einsum("thd,thd->th", q, k), rtol=0, atol=1e-13)


def test_dominant_scores_give_the_hard_maximum_without_overflow():
    # scores up to ~1e6: the softmax must subtract its maximum.  Key u has
    # first feature u, every query is 1e4 e_0 (no rotation), so the latest
    # key u = t wins by 1e4 * scale per step: out_t = v_t, lse = score_t.
    T, H, d = 50, 1, 8
    q = np.zeros((T, H, d))
    q[:, 0, 0] = 1e4
    k = np.zeros((T, H, d))
    k[:, 0, 0] = np.arange(T)
    v = rng(6).standard_normal((T, H, d))
    out, lse = SO.attention(q, k, v, None, rotary_dim=0, scale=1.0)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(out[1:], v[1:], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[:, 0], 1e4 * np.arange(T), rtol=1e-15, atol=1e-9)


def test_grouped_heads_equal_repeated_heads():
    # query head h reads key/value head h // (H / Hkv)
    r = rng(7)
    cu = np.array([0, 30, 64])
    T, H, Hkv, d = 64, 6, 2, 32
    q = r.standard_normal((T, H, d))
    k, v = (r.standard_normal((T, Hkv, d)) for _ in range(2))
    out, lse = SO.attention(q, k, v, cu, rotary_dim=16, rope_base=10000.0)
    out2, lse2 = SO.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), cu,
                              rotary_dim=16, rope_base=10000.0)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_packed_equals_separate_sequences_and_sampled_rows():
    # [Overview] 2.1.3: positions and the causal window restart per sequence
    r = rng(8)
    cu = np.array([0, 17, 17, 50, 51])
    T, H, d = 51, 2, 32
    q, k, v = (r.standard_normal((T, H, d)) for _ in range(3))
    out, lse = SO.attention(q, k, v, cu, rotary_dim=16, rope_base=5e6)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        o1, l1 = SO.attention(q[a:b], k[a:b], v[a:b], None, rotary_dim=16, rope_base=5e6)
        np.testing.assert_array_equal(out[a:b], o1)
        np.testing.assert_array_equal(lse[a:b], l1)
    rows, heads = [50, 3, 20], [1, 0, 1]
    o3, l3 = SO.attention(q, k, v, cu, rotary_dim=16, rope_base=5e6, rows=rows, heads=heads)
    for i, (t, h) in enumerate(zip(rows, heads)):
        np.testing.assert_array_equal(o3[i], out[t, h])
        assert l3[i] == lse[t, h]


def test_rejects_bad_arguments():
    q = np.zeros((4, 2, 8))
    with pytest.raises(ValueError):
        SO.attention(q, np.zeros((4, 3, 8)), np.zeros((4, 3, 8)))   # 3 does not divide 2
    with pytest.raises(ValueError):
        SO.attention(q, q, q, rotary_dim=3)
    with pytest.raises(ValueError):
        SO.attention(q, q, q, np.array([0, 5]))                      # cu past T
