"""GPU parity of the features-given mode (q, k, v arrive as phi(.) already,
e.g. from a projection whose epilogue applies SiLU) against the oracle's
same mode, through the C ABI.

The inputs are arbitrary bf16 feature vectors (the mode does not care how they
were made): N(0, 1) / sqrt(d), and |N(0, 1)| / sqrt(d) for the normalised mode
so that its denominators stay away from zero.  Tolerance: the bf16 bar,
max|err| / rms(ref) <= 1e-2; with bf16-exact features the products are exact
and the measured error is far below it (reported per case).
"""
import numpy as np
import pytest
import torch

from linear_attention_long_amd import api
from oracle import oracle as O
from tests._util import banner, np64, randn, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda"
D = 128


def feats(shape, seed, positive=False):
    x = randn(shape, seed, scale=D ** -0.5)
    return (x.abs() if positive else x).to(torch.bfloat16)


@pytest.mark.parametrize("T,chunk,gated,odt", [(1000, 0, True, torch.float32),
                                                (4101, 1024, True, torch.bfloat16),
                                                (333, 0, False, torch.float32),
                                                (1, 0, False, torch.float32),
                                                (2048, 512, False, torch.float32)])
def test_prefill_features_given(T, chunk, gated, odt):
    banner("featurized prefill T=%d chunk=%d gated=%s out=%s" % (T, chunk, gated, odt))
    H = 4
    q, k, v = (feats((T, H, D), 300 + i) for i in range(3))
    x = randn((T, H * D), 303).to(torch.bfloat16) if gated else None
    S0 = randn((H, D, D), 304, scale=0.05)
    out, S, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), None if x is None else x.to(DEV),
                               state_in=S0.to(DEV), chunk_tokens=chunk, out_dtype=odt,
                               featurized=True)
    torch.cuda.synchronize()
    ref, Sref, _ = O.forward(np64(q), np64(k), np64(v), None if x is None else np64(x),
                             state_in=np64(S0)[None], gated=gated, featurized=True)
    got = np64(out).reshape(T, H * D)
    e_out = rel_err(got, ref)
    e_S = rel_err(np64(S).reshape(H, D, D), Sref[0])
    print("  out %.2e state %.2e" % (e_out, e_S))
    if odt == torch.bfloat16:
        # plus the output's own rounding to bf16, element by element
        rms = np.sqrt(np.mean(ref * ref))
        assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + TOL * rms).all()
    else:
        assert e_out <= TOL
    assert e_S <= TOL


def test_prefill_normalised_features_given():
    banner("featurized prefill normalised T=1500")
    T, H = 1500, 2
    q, k, v = (feats((T, H, D), 310 + i, positive=True) for i in range(3))
    out, S, z = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), normalized=True,
                               chunk_tokens=512, featurized=True)
    torch.cuda.synchronize()
    ref, Sref, zref = O.forward(np64(q), np64(k), np64(v), normalized=True, featurized=True)
    e = rel_err(np64(out).reshape(T, H * D), ref)
    ez = rel_err(np64(z).reshape(H, D), zref[0])
    print("  out %.2e z %.2e" % (e, ez))
    assert e <= TOL and ez <= TOL


def test_varlen_features_given():
    banner("featurized varlen lengths 0,300,1,0,699,64 gated")
    H = 8
    lens = [0, 300, 1, 0, 699, 64]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = (feats((T, H, D), 320 + i) for i in range(3))
    x = randn((T, H * D), 323).to(torch.bfloat16)
    out, S, _ = api.la_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), torch.tensor(cu, device=DEV),
                                      max(lens), x.to(DEV), featurized=True)
    torch.cuda.synchronize()
    ref, Sref, _ = O.forward(np64(q), np64(k), np64(v), np64(x), cu_seqlens=cu, gated=True,
                             featurized=True)
    e, eS = rel_err(np64(out), ref), rel_err(np64(S), Sref)
    print("  out %.2e state %.2e" % (e, eS))
    assert e <= TOL and eS <= TOL


@pytest.mark.parametrize("normalized", [False, True])
def test_decode_features_given(normalized):
    banner("featurized decode normalised=%s" % normalized)
    N, H, steps = 4, 8, 20
    S = randn((N, H, D, D), 330, scale=0.01).to(DEV)
    z = (randn((N, H, D), 331).abs() + 1.0).to(DEV) if normalized else None
    Sr = np64(S)
    zr = None if z is None else np64(z)
    for t in range(steps):
        q, k, v = (feats((N, H, D), 340 + 3 * t + i, positive=normalized) for i in range(3))
        y = api.la_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), S, z, normalized=normalized,
                               featurized=True)
        torch.cuda.synchronize()
        yr, Sr, zr = O.decode_step(np64(q), np64(k), np64(v), Sr, zr, normalized=normalized,
                                   featurized=True)
        assert rel_err(np64(y).reshape(N, H, D), yr) <= 1e-5, t
    assert rel_err(np64(S), Sr) <= 1e-5


def test_prefill_1m_features_given_sampled():
    """The 1M-token workload in the launch configuration bench.py times for this
    mode, its q, k, v values taken as features; sampled outputs (chunk and block
    boundaries, whole 256-token blocks, seeded random tokens) and the final state."""
    from linear_attention_long_amd import inputs
    from tests.test_gpu_zlarge import chunk_tokens, sample_tokens

    w = inputs.WORKLOADS["prefill_1m"]
    banner("prefill_1m workload, features given (sampled)")
    q, k, v, x = inputs.prefill_inputs(w, device="cuda")
    out, S, _ = api.la_prefill(q, k, v, x, featurized=True)
    torch.cuda.synchronize()
    C, dev = chunk_tokens(False, 1, w.T, w.T, w.H, w.d)
    idx = sample_tokens([0], [w.T], C, 4096, 17, every64=dev)
    blocks = np.concatenate([np.arange(256 * b, 256 * (b + 1)) for b in (0, 63, 64, 2048, 4095)])
    idx = np.union1d(idx, blocks).astype(np.int64)
    got = np64(out[0, torch.from_numpy(idx).cuda()])
    S_got = np64(S)
    del out, S
    qc, kc, vc = (t[0].float().cpu() for t in (q, k, v))
    xs = x[0, torch.from_numpy(idx).cuda()].float().cpu()
    del q, k, v, x
    torch.cuda.empty_cache()
    y, S_ref, _ = O.prefill_sampled_f32(qc, kc, vc, idx, featurized=True, nthreads=w.H)
    ref = O.gate(y.reshape(len(idx), w.H * w.d), xs, None, 0, 1e-6)
    e, eS = rel_err(got, ref), rel_err(S_got[0], S_ref[0])
    print("  %d sampled tokens: out %.2e, state %.2e" % (len(idx), e, eS))
    assert e <= TOL and eS <= TOL


def test_serve_step_features_given():
    """One serving step (two decode tokens, two prompt chunks continuing from
    pool rows) with the inputs given as features."""
    banner("featurized serve step: 2 decode tokens + chunks of 100 and 37")
    rows, H = 6, 4
    dslots, pslots, lens = [1, 4], [0, 3], [100, 37]
    nd, total = len(dslots), len(dslots) + sum(lens)
    q, k, v = (feats((total, H, D), 350 + i) for i in range(3))
    x = randn((total, H * D), 353).to(torch.bfloat16)
    pool0 = randn((rows, H, D, D), 354, scale=0.05)
    pool = pool0.to(DEV)
    cu = torch.tensor([0, lens[0], lens[0] + lens[1]], dtype=torch.int32, device=DEV)
    out = api.la_serve_step(q.to(DEV), k.to(DEV), v.to(DEV), pool,
                            torch.tensor(dslots, dtype=torch.int32, device=DEV), cu,
                            torch.tensor(pslots, dtype=torch.int32, device=DEV), max(lens),
                            x.to(DEV), featurized=True)
    torch.cuda.synchronize()
    out = np64(out)
    spans = [(n, n + 1, r) for n, r in enumerate(dslots)]
    a = nd
    for L, r in zip(lens, pslots):
        spans.append((a, a + L, r))
        a += L
    for a, b, r in spans:
        ref, Sref, _ = O.forward(np64(q[a:b]), np64(k[a:b]), np64(v[a:b]), np64(x[a:b]),
                                 state_in=np64(pool0[r:r + 1]), gated=True, featurized=True)
        assert rel_err(out[a:b], ref) <= TOL, (a, b)
        assert rel_err(np64(pool[r]), Sref[0]) <= 1e-4, r


@pytest.mark.parametrize("dtype,d,block", [(torch.float32, 64, 64), (torch.float32, 128, 32),
                                           (torch.bfloat16, 128, 128), (torch.bfloat16, 64, 0)])
def test_vector_path_features_given(dtype, d, block):
    """The fp32 vector path (fp32 inputs, d = 64, blocks of 128 or 256) in the same mode."""
    banner("featurized vector path dtype=%s d=%d block=%d" % (dtype, d, block))
    T, H = 777, 2
    q, k, v = (randn((T, H, d), 360 + i, scale=d ** -0.5).to(dtype) for i in range(3))
    out, S, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), block_size=block,
                               chunk_tokens=256, featurized=True)
    torch.cuda.synchronize()
    ref, Sref, _ = O.forward(np64(q), np64(k), np64(v), featurized=True)
    tol = 1e-5 if dtype == torch.float32 else TOL
    e, eS = rel_err(np64(out).reshape(T, H * d), ref), rel_err(np64(S).reshape(H, d, d), Sref[0])
    print("  out %.2e state %.2e" % (e, eS))
    assert e <= tol and eS <= tol
