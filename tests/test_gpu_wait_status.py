"""The fused gate's bounded waits, and calls on a side stream.

The fused gate makes the H heads of a chunk wait for each other's per-token
sums of y^2 (the RMSNorm of "MiniMax-Text-01 405B MoE模型架构与训练策略解析"
section 2.1 spans all heads of a token).  Every wait is bounded; one that
gives up must never gate with a sum it could not verify.  The failure is
forced from the host (wait_spin_limit = -1: every wait gives up at once), so
every kernel still exits normally.
"""
import ctypes

import numpy as np
import pytest
import torch

from linear_attention_long_amd import _lib, api
from oracle import oracle as O
from tests._util import banner, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"
T, H, D = 2000, 8, 128


def inputs(seed, T=T, H=H):
    g = torch.Generator().manual_seed(seed)
    s = 1.0 / np.sqrt(D)
    q, k, v = ((torch.randn((T, H, D), generator=g) * s).to(torch.bfloat16) for _ in range(3))
    x = torch.randn((T, H * D), generator=g).to(torch.bfloat16)
    return q, k, v, x


def fused_plan(chunk):
    opt = _lib.options(0, False, True, 0, 1e-6, chunk, False)
    p = _lib.plan(False, 1, T, T, H, D, _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32, opt)
    nbytes = _lib.load().la_prefill_workspace_bytes(1, T, H, D, _lib.LA_DTYPE_BF16,
                                                    _lib.LA_DTYPE_F32, ctypes.byref(opt))
    return p, nbytes


@pytest.mark.parametrize("chunk", [512, 2048])   # chunked (scan clears) / one chunk (fill clears)
def test_forced_give_up_poisons_and_reports(chunk):
    banner("wait give-up forced, chunk %d" % chunk)
    p, nbytes = fused_plan(chunk)
    assert p.fused_gate == 1 and p.status_offset >= 0
    q, k, v, x = inputs(41)
    ref, Sref, _ = O.forward(q, k, v, x, gated=True)
    qd, kd, vd, xd = (t.to(DEV) for t in (q, k, v, x))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    # every wait gives up: every gated row is NaN, the status word says so,
    # and the state (which needs no exchange) is still right
    out, S, _ = api.la_prefill(qd, kd, vd, xd, chunk_tokens=chunk, workspace=ws,
                               wait_spin_limit=-1)
    assert api.la_prefill_wait_status(ws, p.status_offset) == _lib.LA_ERR_WAIT_TIMEOUT
    assert bool(torch.isnan(out).all())
    assert rel_err(S.double().cpu().numpy(), Sref[0]) <= 1e-2   # [T, H, d] in: S is [H, d, d]
    # the next call on the same workspace clears the word and gates normally
    out2, S2, _ = api.la_prefill(qd, kd, vd, xd, chunk_tokens=chunk, workspace=ws)
    assert api.la_prefill_wait_status(ws, p.status_offset) == _lib.LA_OK
    assert rel_err(out2.double().cpu().numpy(), ref) <= 1e-2


def test_tiny_spin_limit_never_returns_unverified_rows():
    """With one retry a wait succeeds only if the sums arrive almost at once;
    whatever happens, a finite row is a verified one."""
    banner("wait spin limit 1")
    p, nbytes = fused_plan(512)
    q, k, v, x = inputs(43)
    ref, _, _ = O.forward(q, k, v, x, gated=True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out, _, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), chunk_tokens=512,
                               workspace=ws, wait_spin_limit=1)
    st = api.la_prefill_wait_status(ws, p.status_offset)
    got = out.double().cpu().numpy()
    bad_rows = np.isnan(got).any(axis=1)
    if st == _lib.LA_OK:
        assert not bad_rows.any()
    else:
        assert st == _lib.LA_ERR_WAIT_TIMEOUT and bad_rows.any()
    good = ~bad_rows
    if good.any():
        rms = np.sqrt(np.mean(ref ** 2))
        assert np.abs(got[good] - ref[good]).max() / rms <= 1e-2
    print("spin limit 1: status %d, %d of %d rows poisoned" % (st, bad_rows.sum(), T))


def test_plan_without_wait_has_no_status_word():
    opt = _lib.options(0, False, False, 0, 1e-6, 0, False)  # ungated: no exchange
    p = _lib.plan(False, 1, T, T, H, D, _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32, opt)
    assert p.fused_gate == 0 and p.status_offset == -1
    assert api.la_prefill_wait_status(None, -1) == _lib.LA_OK


def test_calls_on_a_side_stream():
    """la_prefill, la_prefill_varlen and la_decode_step enqueued on a stream
    other than the current one; the current stream then allocates and writes
    fresh memory while that work may still run (the caching allocator must
    not hand it the calls' buffers), then both are compared with the oracle."""
    banner("side stream")
    q, k, v, x = inputs(45, T=1500)
    ref, Sref, _ = O.forward(q, k, v, x, gated=True)
    qd, kd, vd, xd = (t.to(DEV) for t in (q, k, v, x))
    cu = torch.tensor([0, 700, 700, 1500], dtype=torch.int32, device=DEV)
    qs, ks, vs = (t[:4].contiguous() for t in (qd, kd, vd))
    S0 = np.repeat(Sref, 4, axis=0)
    Sdec = torch.from_numpy(S0).float().to(DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())  # inputs are ready
    out, S, _ = api.la_prefill(qd, kd, vd, xd, chunk_tokens=256, stream=side)
    outv, Sv, _ = api.la_prefill_varlen(qd, kd, vd, cu, 800, xd, stream=side)
    y = api.la_decode_step(qs, ks, vs, Sdec, stream=side)
    junk = [torch.full((1 << 20,), float(i), device=DEV) for i in range(16)]
    side.synchronize()
    torch.cuda.synchronize()
    assert all(float(j[0]) == i for i, j in enumerate(junk))
    assert rel_err(out.double().cpu().numpy(), ref) <= 1e-2
    assert rel_err(S.double().cpu().numpy(), Sref[0]) <= 1e-2
    cuh = cu.cpu().numpy()
    refv, Svref, _ = O.forward(q, k, v, x, cu_seqlens=cuh, gated=True)
    assert rel_err(outv.double().cpu().numpy(), refv) <= 1e-2
    assert rel_err(Sv.double().cpu().numpy(), Svref) <= 1e-2
    yref, _, _ = O.decode_step(q[:4], k[:4], v[:4], S0)
    assert rel_err(y.double().cpu().numpy(), yref.reshape(4, H * D)) <= 1e-2
