"""GPU parity of the layer's input projection (include/la_proj.h) against its
CPU oracle (oracle/projection.py), and of the projection followed by the
attention path against the oracles chained the same way.

Page "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1: Q, K, V =
SiLU of the layer input's projections; the gate sigmoid(.) of a projection of
its own.

Tolerances.  The inputs are bf16 and the products are exact in fp32, so an
fp32 output differs from the fp64 oracle only by the fp32 accumulation over
K: at most 1e-4 of the output's rms here (an implementation check; it
measures ~1e-6).  A bf16 output is additionally rounded once, to 8
significant bits: each element within half a bf16 ulp of the oracle's value
(at most 2^-8 of its magnitude) plus the accumulation term.
"""
import numpy as np
import pytest
import torch

from linear_attention_long_amd import api
from oracle import oracle as O
from oracle import projection as P
from tests._util import banner, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


def make(T, K, F, seed, nblk=4):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn((T, K), generator=g).to(torch.bfloat16)
    # weight scaled so the projections are O(1) (unit-variance rows of h)
    w = (torch.randn((nblk * F, K), generator=g) / np.sqrt(K)).to(torch.bfloat16)
    return h, w


def check_f32(got, ref):
    e = rel_err(got, ref)
    assert e <= 1e-4, e
    return e


def check_bf16(got, ref):
    rms = np.sqrt(np.mean(ref * ref))
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * rms
    bad = np.abs(got - ref) > bound
    assert not bad.any(), "%d elements outside the bf16 storage bound" % bad.sum()


# T = 1537: 7 token tiles, a full group of 4 in the tile order and a partial
# group of 3
@pytest.mark.parametrize("T,K,F", [(1, 64, 256), (255, 128, 256), (257, 320, 512),
                                   (1000, 6144, 1024), (1537, 256, 1024)])
@pytest.mark.parametrize("featurize", [True, False])
def test_projection_fp32_out(T, K, F, featurize):
    banner("projection T=%d K=%d F=%d featurize=%s fp32 out" % (T, K, F, featurize))
    h, w = make(T, K, F, 10 + T)
    got = api.la_qkvx_projection(h.to(DEV), w.to(DEV), F, featurize=featurize,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = P.project(h, w, F, featurize=featurize)
    for a, b in zip(got, ref):
        check_f32(a.double().cpu().numpy(), b)


@pytest.mark.parametrize("T,gate", [(300, True), (513, False), (4096, True)])
def test_projection_bf16_out(T, gate):
    K, F = 6144, 1024
    banner("projection T=%d bf16 out gate=%s" % (T, gate))
    nblk = 4 if gate else 3
    h, w = make(T, K, F, 20 + T, nblk)
    got = api.la_qkvx_projection(h.to(DEV), w.to(DEV), F, gate=gate)
    torch.cuda.synchronize()
    if not gate:
        assert got[3] is None
        w4 = torch.cat([w, torch.zeros((F, K), dtype=w.dtype)])
    else:
        w4 = w
    ref = P.project(h, w4, F)
    for a, b in zip(got[:nblk], ref[:nblk]):
        check_bf16(a.double().cpu().numpy(), b)


def test_projection_32k_sampled_rows():
    """The benched shape (T = 32768, K = 6144, F = 1024): sampled token rows
    (first and last of tiles, the very first and last tokens, random rows)
    of all four outputs, and the untouched guard around the outputs."""
    T, K, F = 32768, 6144, 1024
    banner("projection 32K sampled")
    h, w = make(T, K, F, 31)
    outs = [torch.full((T + 64, F), float("nan"), dtype=torch.bfloat16, device=DEV)
            for _ in range(4)]
    got = api.la_qkvx_projection(h.to(DEV), w.to(DEV), F, out=[o[32:32 + T] for o in outs])
    torch.cuda.synchronize()
    for o in outs:  # nothing written outside the views
        assert bool(torch.isnan(o[:32]).all()) and bool(torch.isnan(o[32 + T:]).all())
    r = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 255, 256, 511, T - 257, T - 256, T - 1],
                                     r.integers(0, T, 200)]))
    ref = P.project(h, w, F, rows=rows)
    ri = torch.from_numpy(rows).to(DEV)
    for a, b in zip(got, ref):
        check_bf16(a[ri].double().cpu().numpy(), b)


@pytest.mark.parametrize("featurize", [True, False])
def test_projection_then_path(featurize):
    """The layer from its input: projection (SiLU in the epilogue, then the
    path in its features-given mode; or raw projections, then the path's own
    SiLU) against the oracles chained the same way: the projection in fp64,
    its outputs rounded to bf16 as they are stored, then the path oracle."""
    T, K, H, d = 1500, 1024, 8, 128
    F = H * d
    banner("projection then path, featurize=%s" % featurize)
    h, w = make(T, K, F, 41)
    q, k, v, xg = api.la_qkvx_projection(h.to(DEV), w.to(DEV), F, featurize=featurize)
    out, S, _ = api.la_prefill(q.view(T, H, d), k.view(T, H, d), v.view(T, H, d), xg,
                               chunk_tokens=512, featurized=featurize)
    torch.cuda.synchronize()
    pq, pk, pv, px = (torch.from_numpy(a).to(torch.bfloat16)
                      for a in P.project(h, w, F, featurize=featurize))
    ref, Sref, _ = O.forward(pq.view(T, H, d), pk.view(T, H, d), pv.view(T, H, d), px,
                             gated=True, featurized=featurize)
    e, es = rel_err(out.double().cpu().numpy(), ref), rel_err(S.double().cpu().numpy(), Sref[0])
    print("projection then path (featurize=%s): out %.2e state %.2e" % (featurize, e, es))
    assert e <= 1e-2 and es <= 1e-2


def test_projection_1m_workload_sampled():
    """The bench's 1M-token projection (hidden [1048576, 6144] drawn on the GPU
    as the bench draws it): sampled rows, including the first and last tokens
    and tile edges, of all four outputs."""
    from linear_attention_long_amd import inputs

    w = inputs.WORKLOADS["proj_1m"]
    banner("projection 1M sampled")
    h, wt = inputs.projection_inputs(w, device=DEV)
    T, F = h.shape[0], w.H * w.d
    got = api.la_qkvx_projection(h, wt, F)
    torch.cuda.synchronize()
    r = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, T // 2, T - 257, T - 256, T - 1],
                                     r.integers(0, T, 120)]))
    ri = torch.from_numpy(rows).to(DEV)
    ref = P.project(h[ri].cpu(), wt.cpu(), F)
    for a, b in zip(got, ref):
        check_bf16(a[ri].double().cpu().numpy(), b)
    del h, got
    torch.cuda.empty_cache()


# ---- the output projection (la_out_projection): y [T, K] bf16 times W_o [N, K]^T ----


def make_out(T, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    y = torch.randn((T, K), generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g) / np.sqrt(K)).to(torch.bfloat16)
    return y, w


@pytest.mark.parametrize("T,K,N", [(1, 64, 256), (255, 128, 512), (257, 1024, 6144),
                                   (1000, 1024, 6144), (1537, 256, 768)])
def test_out_projection_fp32_out(T, K, N):
    banner("out projection T=%d K=%d N=%d fp32 out" % (T, K, N))
    y, w = make_out(T, K, N, 50 + T)
    got = api.la_out_projection(y.to(DEV), w.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_f32(got.double().cpu().numpy(), P.out_project(y, w))


@pytest.mark.parametrize("T", [300, 4096])
def test_out_projection_bf16_out(T):
    K, N = 1024, 6144
    banner("out projection T=%d bf16 out" % T)
    y, w = make_out(T, K, N, 60 + T)
    got = api.la_out_projection(y.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    check_bf16(got.double().cpu().numpy(), P.out_project(y, w))


def test_out_projection_32k_sampled_rows():
    """The benched shape (T = 32768, K = 1024, N = 6144): sampled rows, and
    the untouched guard around the output."""
    T, K, N = 32768, 1024, 6144
    banner("out projection 32K sampled")
    y, w = make_out(T, K, N, 71)
    buf = torch.full((T + 64, N), float("nan"), dtype=torch.float32, device=DEV)
    got = api.la_out_projection(y.to(DEV), w.to(DEV), out=buf[32:32 + T])
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf[:32]).all()) and bool(torch.isnan(buf[32 + T:]).all())
    r = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 255, 256, 511, T - 257, T - 256, T - 1],
                                     r.integers(0, T, 200)]))
    ri = torch.from_numpy(rows).to(DEV)
    check_f32(got[ri].double().cpu().numpy(), P.out_project(y, w, rows=rows))


def test_whole_layer_projections_and_path():
    """The layer from its input to its output on one device's heads: input
    projection (SiLU in the epilogue), the path in its features-given mode
    with the gate and bf16 output, then the output projection -- against the
    oracles chained the same way (fp64 at every step, the tensors rounded to
    bf16 where the device stores them in bf16)."""
    T, K, H, d, N = 1500, 1024, 8, 128, 2048
    F = H * d
    banner("whole layer: projection, path, output projection")
    h, w = make(T, K, F, 81)
    _, wo = make_out(1, F, N, 82)
    q, k, v, xg = api.la_qkvx_projection(h.to(DEV), w.to(DEV), F)
    y, _, _ = api.la_prefill(q.view(T, H, d), k.view(T, H, d), v.view(T, H, d), xg,
                             chunk_tokens=512, featurized=True, out_dtype=torch.bfloat16,
                             return_state=False)
    z = api.la_out_projection(y.view(T, F), wo.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    pq, pk, pv, px = (torch.from_numpy(a).to(torch.bfloat16) for a in P.project(h, w, F))
    yref, _, _ = O.forward(pq.view(T, H, d), pk.view(T, H, d), pv.view(T, H, d), px,
                           gated=True, featurized=True)
    yref16 = torch.from_numpy(yref).to(torch.bfloat16)
    zref = P.out_project(yref16, wo)
    e = rel_err(z.double().cpu().numpy(), zref)
    print("whole layer: output %.2e of rms" % e)
    assert e <= 1e-2


def test_out_projection_1m_workload_sampled():
    """The bench's 1M-token output side (y [1048576, 1024] and W_o [6144,
    1024] drawn on the GPU as the bench draws them), bf16 output: sampled
    rows, including the first and last tokens and tile edges."""
    from linear_attention_long_amd import inputs

    w = inputs.WORKLOADS["proj_1m"]
    banner("out projection 1M sampled")
    y, wo = inputs.out_projection_inputs(w, device=DEV)
    T = y.shape[0]
    z = api.la_out_projection(y, wo)
    torch.cuda.synchronize()
    r = np.random.default_rng(10)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, T // 2, T - 257, T - 256, T - 1],
                                     r.integers(0, T, 120)]))
    ri = torch.from_numpy(rows).to(DEV)
    check_bf16(z[ri].double().cpu().numpy(), P.out_project(y[ri].cpu(), wo.cpu()))
    del y, z
    torch.cuda.empty_cache()
