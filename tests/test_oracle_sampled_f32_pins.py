"""Pins of the oracle's float-input sampled recurrence (``prefill_sampled_f32``).

This is the reference of every parity test too large for fp64 outputs (the
1M- and 4M-token prefills, the packed 512K batch, the 1000-step decode chain,
the features-given 1M prefill), so its own plumbing is pinned here on the CPU:
the widening of float inputs one token at a time, the per-token offsets into
q, k and v, sampling across sequence boundaries (duplicate indices, the first
and last token of every sequence, tokens either side of every boundary),
empty sequences, and per-sequence ``state_in`` / ``z_in``.

Two references, neither of which goes through this function's code:

* the brute-force masked quadratic form of "六十四：MiniMax-01" section 3
  (sum over i <= t of (phi(q_t).phi(k_i)) phi(v_i), plus phi(q_t) S0 for a
  carried state), evaluated per sequence with numpy matmuls and a tanh-based
  SiLU, and the closed-form final state S0 + phi(K)^T phi(V);
* the fp64 recurrence ``prefill`` (itself pinned in ``test_oracle_pins.py``)
  on the same values widened up front: the widening is exact, so the two must
  agree bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O


def silu_tanh(x):
    return x * 0.5 * (1.0 + np.tanh(0.5 * x))


def rel(a, b):
    return np.abs(a - b).max() / max(np.sqrt(np.mean(b ** 2)), 1e-300)


def masked_form(q, k, v, S0, z0, normalized, featurized):
    """One sequence [L, H, d] in fp64: tril(A B^T) C + A S0 per head (and the
    normalised ratio over tril(A B^T) 1 + A z0)."""
    f = (lambda x: x) if featurized else silu_tanh
    a, b, c = f(q), f(k), f(v)
    L, H, d = q.shape
    y = np.zeros((L, H, d))
    S = np.zeros((H, d, d))
    z = np.zeros((H, d))
    for h in range(H):
        P = np.tril(a[:, h] @ b[:, h].T)
        num = P @ c[:, h] + a[:, h] @ S0[h]
        S[h] = S0[h] + b[:, h].T @ c[:, h]
        z[h] = z0[h] + b[:, h].sum(axis=0)
        if normalized:
            num = num / (P.sum(axis=1) + a[:, h] @ z0[h])[:, None]
        y[:, h] = num
    return y, S, z


def boundary_samples(cu, rng, extra=6):
    """Sorted sample indices: first and last token of every non-empty
    sequence, the tokens on each side of every boundary, duplicates, and a few
    random tokens."""
    total = int(cu[-1])
    idx = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            idx += [a, b - 1, a, b - 1]          # first/last, each twice
        for t in (a - 1, a, b - 1, b):           # either side of both edges
            if 0 <= t < total:
                idx.append(t)
    idx += list(rng.integers(0, total, size=extra))
    return np.sort(np.array(idx, dtype=np.int64))


# lengths with empty sequences at the start, in the middle and at the end
LENGTHS = [0, 7, 1, 0, 40, 3, 0, 25, 0]


def make_case(seed, dtype, normalized, featurized):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int64)
    total, H, d, nseq = int(cu[-1]), 3, 16, len(LENGTHS)
    g = torch.Generator().manual_seed(seed)
    sh = 1.5 if normalized else 0.0   # keeps phi(q).z away from zero
    q, k, v = ((torch.randn((total, H, d), generator=g) * 0.7 + sh).to(dtype) for _ in range(3))
    S0 = np.abs(rng.standard_normal((nseq, H, d, d))) * 0.05
    z0 = np.abs(rng.standard_normal((nseq, H, d))) + 0.5
    return cu, q, k, v, S0, z0, rng


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("normalized", [False, True])
@pytest.mark.parametrize("featurized", [False, True])
def test_sampled_f32_equals_masked_form_and_fp64(dtype, normalized, featurized):
    seed = 300 + 4 * int(normalized) + 2 * int(featurized) + (dtype == torch.float32)
    cu, q, k, v, S0, z0, rng = make_case(seed, dtype, normalized, featurized)
    idx = boundary_samples(cu, rng)
    zin = z0 if normalized else None
    y, S, z = O.prefill_sampled_f32(q, k, v, idx, cu_seqlens=cu, state_in=S0, z_in=zin,
                                    normalized=normalized, featurized=featurized)
    # bit for bit the fp64 recurrence on the same (exactly widened) values
    yd, Sd, zd = O.prefill(q, k, v, cu_seqlens=cu, state_in=S0, z_in=zin, normalized=normalized,
                           featurized=featurized, sample_idx=idx)
    assert np.array_equal(y, yd)
    assert np.array_equal(S, Sd)
    assert np.array_equal(z, zd)
    # the masked quadratic form per sequence, at every sampled token
    qd, kd, vd = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    zref0 = z0 if normalized else np.zeros_like(z0)
    for s in range(len(LENGTHS)):
        a, b = int(cu[s]), int(cu[s + 1])
        ys, Ss, zs = masked_form(qd[a:b], kd[a:b], vd[a:b], S0[s], zref0[s], normalized,
                                 featurized)
        rows = np.nonzero((idx >= a) & (idx < b))[0]
        if len(rows):
            assert rel(y[rows], ys[idx[rows] - a]) < 1e-12, s
        # final state: the closed form (an empty sequence keeps its state)
        assert np.abs(S[s] - Ss).max() < 1e-12 * max(1.0, np.abs(Ss).max()), s
        if normalized:
            assert np.abs(z[s] - zs).max() < 1e-12 * max(1.0, np.abs(zs).max()), s


def test_sampled_f32_without_state_starts_from_zero():
    """No state_in: every sequence starts from S = 0 (the masked form with
    S0 = 0); duplicate indices receive identical rows."""
    cu, q, k, v, S0, z0, rng = make_case(331, torch.bfloat16, False, False)
    idx = boundary_samples(cu, rng)
    y, S, _ = O.prefill_sampled_f32(q, k, v, idx, cu_seqlens=cu)
    qd, kd, vd = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    for s in range(len(LENGTHS)):
        a, b = int(cu[s]), int(cu[s + 1])
        ys, Ss, _ = masked_form(qd[a:b], kd[a:b], vd[a:b], np.zeros_like(S0[s]),
                                np.zeros_like(z0[s]), False, False)
        rows = np.nonzero((idx >= a) & (idx < b))[0]
        if len(rows):
            assert rel(y[rows], ys[idx[rows] - a]) < 1e-12
        assert np.abs(S[s] - Ss).max() < 1e-12 * max(1.0, np.abs(Ss).max())
    for i in range(1, len(idx)):
        if idx[i] == idx[i - 1]:
            assert np.array_equal(y[i], y[i - 1])


def test_sampled_f32_single_sequence_and_last_token():
    """One sequence without cu_seqlens; the last token's output equals the
    non-causal phi(q_T) (phi(K)^T phi(V)) ([Arch] section 2.1's Q (K^T V))."""
    g = torch.Generator().manual_seed(333)
    T, H, d = 97, 2, 32
    q, k, v = ((torch.randn((T, H, d), generator=g) * 0.5).to(torch.bfloat16) for _ in range(3))
    idx = np.array([0, 31, 32, 33, 95, 96, 96], dtype=np.int64)
    y, S, _ = O.prefill_sampled_f32(q, k, v, idx)
    a, b, c = (silu_tanh(t.float().numpy().astype(np.float64)) for t in (q, k, v))
    for h in range(H):
        KV = b[:, h].T @ c[:, h]
        assert np.abs(y[-1, h] - a[-1, h] @ KV).max() < 1e-12 * np.abs(a[-1, h] @ KV).max()
        assert np.abs(S[0, h] - KV).max() < 1e-12 * np.abs(KV).max()
    assert np.array_equal(y[-1], y[-2])


def test_sampled_f32_rejects_bad_indices():
    g = torch.Generator().manual_seed(335)
    q = torch.randn((10, 1, 8), generator=g)
    with pytest.raises(ValueError):
        O.prefill_sampled_f32(q, q, q, np.array([3, 2]))       # not sorted
    with pytest.raises(ValueError):
        O.prefill_sampled_f32(q, q, q, np.array([0, 10]))      # past the end
