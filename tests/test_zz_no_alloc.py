"""la_prefill_noalloc: the prefill entry point that allocates nothing (its
scratch is the library's fixed per-GPU array), for callers that cannot call
hipMalloc.  Checked through the C ABI against la_prefill with a caller
workspace -- the same kernels, so the outputs must agree bit for bit -- and
against the oracle at the bf16 bound (1e-2 of rms), on two calls in a row,
the second smaller than the first (the array keeps the first call's
contents, which the second must not depend on)."""
import ctypes

import numpy as np
import pytest
import torch

from linear_attention_long_amd import _lib, api
from oracle import oracle as O
from tests._util import banner, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16, F32 = _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32


def case(T, H, seed, gated):
    g = torch.Generator().manual_seed(seed)
    s = 1.0 / np.sqrt(128)
    q, k, v = ((torch.randn((1, T, H, 128), generator=g) * s).to(torch.bfloat16) for _ in range(3))
    x = torch.randn((1, T, H * 128), generator=g).to(torch.bfloat16) if gated else None
    return q, k, v, x


def p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc_call(q, k, v, x, opt, out, so):
    _, T, H, d = q.shape
    st = _lib.load().la_prefill_noalloc(p(q), p(k), p(v), p(x), None, None, None, p(out), p(so),
                                        None, 1, T, H, d, BF16, F32, ctypes.byref(opt),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("first,second", [((3000, 8, True, 512), (700, 8, True, 256)),
                                          ((5000, 4, False, 1024), (1000, 4, False, 0))])
def test_noalloc_equals_workspace_call(first, second):
    for (T, H, gated, chunk), seed in ((first, 11), (second, 12)):
        banner("noalloc T=%d H=%d gated=%s chunk=%d" % (T, H, gated, chunk))
        q, k, v, x = case(T, H, seed, gated)
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        xd = None if x is None else x.to(DEV)
        opt = _lib.options(gated=gated, chunk_tokens=chunk)
        out = torch.full((1, T, H * 128), float("nan"), device=DEV)
        so = torch.full((1, H, 128, 128), float("nan"), device=DEV)
        assert noalloc_call(qd, kd, vd, xd, opt, out, so) == _lib.LA_OK
        ref_out, ref_S, _ = api.la_prefill(qd, kd, vd, xd, chunk_tokens=chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(so, ref_S)
        o64, S64, _ = O.forward(q[0], k[0], v[0], None if x is None else x[0], gated=gated)
        assert rel_err(out[0].double().cpu().numpy(), o64) <= 1e-2
        assert rel_err(so[0].double().cpu().numpy(), S64[0]) <= 1e-2


def test_noalloc_rejects_a_plan_beyond_its_scratch():
    """1M tokens x 8 heads ungated needs 128 MiB of chunk states: refused on
    the host, nothing launched, the output untouched."""
    lib = _lib.load()
    T, H = 1 << 20, 8
    opt = _lib.options()
    need = lib.la_prefill_workspace_bytes(1, T, H, 128, BF16, F32, ctypes.byref(opt))
    assert need > _lib.LA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((1, T, H, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.full((1, T, H * 128), 7.0, device=DEV)
    assert noalloc_call(q, q, q, None, opt, out, None) == _lib.LA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_falls_back_to_whole_chunk_state_pass_when_half_chunks_do_not_fit():
    """A gated 524,288-token call: with a caller workspace the plan runs the
    chunk-state pass on half chunks, whose partial increments push it past the
    fixed array; the entry point then plans the state pass on whole chunks,
    which fits.  The two plans round the chunk prefixes in different orders,
    so the outputs agree to fp32 accumulation (held to 1e-4 of rms), not bit
    for bit."""
    lib = _lib.load()
    T, H = 1 << 19, 8
    banner("noalloc fallback T=%d H=%d gated" % (T, H))
    opt = _lib.options(gated=True)
    need = lib.la_prefill_workspace_bytes(1, T, H, 128, BF16, F32, ctypes.byref(opt))
    assert need > _lib.LA_NOALLOC_SCRATCH_BYTES
    g = torch.Generator(device=DEV).manual_seed(21)
    s = 1.0 / np.sqrt(128)
    q, k, v = ((torch.randn((1, T, H, 128), generator=g, device=DEV) * s).to(torch.bfloat16)
               for _ in range(3))
    x = torch.randn((1, T, H * 128), generator=g, device=DEV).to(torch.bfloat16)
    out = torch.full((1, T, H * 128), float("nan"), device=DEV)
    so = torch.full((1, H, 128, 128), float("nan"), device=DEV)
    assert noalloc_call(q, k, v, x, opt, out, so) == _lib.LA_OK
    ref_out, ref_S, _ = api.la_prefill(q, k, v, x)
    torch.cuda.synchronize()
    err = float((out - ref_out).abs().max() / ref_out.pow(2).mean().sqrt())
    serr = float((so - ref_S).abs().max() / ref_S.pow(2).mean().sqrt())
    print("noalloc whole-chunk plan against the half-chunk plan: out %.2e, state %.2e of rms" % (err, serr))
    assert err <= 1e-4 and serr <= 1e-4
