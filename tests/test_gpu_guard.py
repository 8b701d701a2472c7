"""Every output of every entry point, poisoned and fenced: each output buffer
is a view into a larger allocation filled with a NaN bit pattern, with 4 KiB
guard bands before and after it.  After the call every element of the view
must be finite (nothing left unwritten) and every guard byte unchanged
(nothing written out of bounds).  Parity itself is tested elsewhere; these
tests check coverage and bounds of the writes, on ragged shapes: tails that
are not a multiple of any block, empty and one-token sequences, chunked
sequences, bf16 and fp32 outputs, in-place state updates.
"""
import ctypes

import numpy as np
import pytest
import torch

from linear_attention_long_amd import _lib, api

pytestmark = pytest.mark.gpu

DEV = "cuda"
GUARD = 4096  # bytes on each side
PAT32 = 0x7FBADBAD  # a NaN as fp32
PAT16 = 0x7FBB      # a NaN as bf16


class Fenced:
    """A tensor of `shape`/`dtype` inside NaN-filled memory with guard bands."""

    def __init__(self, shape, dtype, init=None):
        self.shape, self.dtype = tuple(shape), dtype
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(self.shape))
        self.g = GUARD // esz
        if dtype == torch.bfloat16:
            raw = torch.full((n + 2 * self.g,), PAT16, dtype=torch.int16, device=DEV)
            self.buf = raw.view(torch.bfloat16)
        else:
            raw = torch.full((n + 2 * self.g,), PAT32, dtype=torch.int32, device=DEV)
            self.buf = raw.view(dtype)
        self.raw = raw
        self.t = self.buf[self.g:self.g + n].view(self.shape)
        if init is not None:
            self.t.copy_(init)
        self.head = raw[:self.g].clone()
        self.tail = raw[self.g + n:].clone()

    def check(self, name, written=None):
        torch.cuda.synchronize()
        n = int(np.prod(self.shape))
        assert torch.equal(self.raw[:self.g], self.head), "%s: write before the buffer" % name
        assert torch.equal(self.raw[self.g + n:], self.tail), "%s: write past the buffer" % name
        t = self.t if written is None else written(self.t)
        bad = int((~torch.isfinite(t.float())).sum())
        assert bad == 0, "%s: %d elements left unwritten (NaN)" % (name, bad)


def rnd(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(dtype)


def ws(nbytes):
    return None if nbytes in (0, ctypes.c_size_t(-1).value) else torch.empty(
        nbytes, dtype=torch.uint8, device=DEV)


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("T,chunk,gated,odt", [(1000, 256, True, torch.float32),
                                                 (1000, 0, True, torch.bfloat16),
                                                 (333, 0, False, torch.float32),
                                                 (4101, 1024, False, torch.bfloat16)])
def test_prefill_writes_exactly_its_outputs(T, chunk, gated, odt):
    lib = _lib.load()
    Bt, H, d = 2, 4, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (rnd((Bt, T, H, d), i, s) for i in range(3))
    x = rnd((Bt, T, H * d), 3) if gated else None
    out = Fenced((Bt, T, H * d), odt)
    so = Fenced((Bt, H, d, d), torch.float32)
    opt = _lib.options(gated=gated, chunk_tokens=chunk)
    in_dt, out_dt = _lib.LA_DTYPE_BF16, (_lib.LA_DTYPE_BF16 if odt == torch.bfloat16
                                         else _lib.LA_DTYPE_F32)
    w = ws(lib.la_prefill_workspace_bytes(Bt, T, H, d, in_dt, out_dt, ctypes.byref(opt)))
    st = lib.la_prefill(ptr(q), ptr(k), ptr(v), ptr(x), None, None, None, ptr(out.t), ptr(so.t),
                        None, Bt, T, H, d, in_dt, out_dt, ctypes.byref(opt), ptr(w),
                        0 if w is None else w.numel(), stream())
    _lib.check(st, "la_prefill")
    out.check("out")
    so.check("state_out")


@pytest.mark.parametrize("T,chunk,gated,odt", [(1000, 256, True, torch.float32),
                                                 (4101, 1024, False, torch.bfloat16)])
def test_prefill_features_given_writes_exactly_its_outputs(T, chunk, gated, odt):
    lib = _lib.load()
    Bt, H, d = 2, 4, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (rnd((Bt, T, H, d), 50 + i, s) for i in range(3))
    x = rnd((Bt, T, H * d), 53) if gated else None
    out = Fenced((Bt, T, H * d), odt)
    so = Fenced((Bt, H, d, d), torch.float32)
    opt = _lib.options(gated=gated, chunk_tokens=chunk, featurized=True)
    in_dt, out_dt = _lib.LA_DTYPE_BF16, (_lib.LA_DTYPE_BF16 if odt == torch.bfloat16
                                         else _lib.LA_DTYPE_F32)
    w = ws(lib.la_prefill_workspace_bytes(Bt, T, H, d, in_dt, out_dt, ctypes.byref(opt)))
    st = lib.la_prefill(ptr(q), ptr(k), ptr(v), ptr(x), None, None, None, ptr(out.t), ptr(so.t),
                        None, Bt, T, H, d, in_dt, out_dt, ctypes.byref(opt), ptr(w),
                        0 if w is None else w.numel(), stream())
    _lib.check(st, "la_prefill")
    out.check("out")
    so.check("state_out")


def test_prefill_varlen_normalised_writes_exactly_its_outputs():
    lib = _lib.load()
    H, d = 2, 128
    lens = [0, 300, 1, 0, 699, 64]
    T = sum(lens)
    s = 1.0 / np.sqrt(d)
    q, k, v = (rnd((T, H, d), 10 + i, s) for i in range(3))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    out = Fenced((T, H * d), torch.float32)
    so = Fenced((len(lens), H, d, d), torch.float32)
    zo = Fenced((len(lens), H, d), torch.float32)
    opt = _lib.options(normalized=True, chunk_tokens=128)
    w = ws(lib.la_prefill_varlen_workspace_bytes(T, len(lens), 699, H, d, _lib.LA_DTYPE_BF16,
                                                 _lib.LA_DTYPE_F32, ctypes.byref(opt)))
    st = lib.la_prefill_varlen(ptr(q), ptr(k), ptr(v), None, None, ptr(cu), len(lens), T, 699,
                               None, None, ptr(out.t), ptr(so.t), ptr(zo.t), H, d,
                               _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32, ctypes.byref(opt), ptr(w),
                               0 if w is None else w.numel(), stream())
    _lib.check(st, "la_prefill_varlen")
    out.check("out")
    # every sequence, empty ones included, gets a final state (zeros)
    so.check("state_out")
    zo.check("z_out")


@pytest.mark.parametrize("gated,odt", [(False, torch.float32), (True, torch.bfloat16)])
def test_decode_writes_exactly_its_outputs(gated, odt):
    N, H, d = 5, 3, 128
    q, k, v = (rnd((N, H, d), 20 + i, 0.1) for i in range(3))
    x = rnd((N, H * d), 23) if gated else None
    S = Fenced((N, H, d, d), torch.float32, init=rnd((N, H, d, d), 24, 0.01, torch.float32))
    out = Fenced((N, H * d), odt)
    api.la_decode_step(q, k, v, S.t, x=x, out=out.t, out_dtype=odt)
    out.check("out")
    S.check("state (in place)")


@pytest.mark.parametrize("precision,odt", [(0, torch.bfloat16), (0, torch.float32),
                                           (1, torch.float32), (2, torch.bfloat16)])
def test_softmax_writes_exactly_its_outputs(precision, odt):
    lib = _lib.load()
    H, Hkv, d = 4, 2, 128
    lens = [0, 1, 255, 256, 257, 0, 1000]
    T = sum(lens)
    q, k, v = rnd((T, H, d), 30), rnd((T, Hkv, d), 31), rnd((T, Hkv, d), 32)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    out = Fenced((T, H, d), odt)
    lse = Fenced((T, H), torch.float32)
    opt = _lib.softmax_options(precision=precision)
    out_dt = _lib.LA_DTYPE_BF16 if odt == torch.bfloat16 else _lib.LA_DTYPE_F32
    w = ws(lib.la_softmax_workspace_bytes(len(lens), T, 1000, H, Hkv, d, _lib.LA_DTYPE_BF16,
                                          out_dt, ctypes.byref(opt)))
    st = lib.la_softmax_attention_varlen(ptr(q), ptr(k), ptr(v), ptr(cu), len(lens), T, 1000, H,
                                         Hkv, d, _lib.LA_DTYPE_BF16, out_dt, ptr(out.t),
                                         ptr(lse.t), ctypes.byref(opt), ptr(w),
                                         0 if w is None else w.numel(), stream())
    _lib.check(st, "la_softmax_attention_varlen")
    out.check("out")
    lse.check("lse")


def test_fp32_prefill_writes_exactly_its_outputs():
    lib = _lib.load()
    Bt, T, H, d = 1, 777, 2, 64
    q, k, v = (rnd((Bt, T, H, d), 40 + i, 1.0, torch.float32) for i in range(3))
    out = Fenced((Bt, T, H * d), torch.float32)
    so = Fenced((Bt, H, d, d), torch.float32)
    opt = _lib.options(chunk_tokens=256)
    w = ws(lib.la_prefill_workspace_bytes(Bt, T, H, d, _lib.LA_DTYPE_F32, _lib.LA_DTYPE_F32,
                                          ctypes.byref(opt)))
    st = lib.la_prefill(ptr(q), ptr(k), ptr(v), None, None, None, None, ptr(out.t), ptr(so.t),
                        None, Bt, T, H, d, _lib.LA_DTYPE_F32, _lib.LA_DTYPE_F32,
                        ctypes.byref(opt), ptr(w), 0 if w is None else w.numel(), stream())
    _lib.check(st, "la_prefill")
    out.check("out")
    so.check("state_out")


@pytest.mark.parametrize("T,odt,gate", [(1, torch.bfloat16, True), (257, torch.float32, True),
                                        (300, torch.bfloat16, False)])
def test_input_projection_writes_exactly_its_outputs(T, odt, gate):
    K, F = 320, 512
    h = rnd((T, K), 40)
    nblk = 4 if gate else 3
    w = rnd((nblk * F, K), 41, K ** -0.5)
    outs = [Fenced((T, F), odt) for _ in range(nblk)]
    api.la_qkvx_projection(h, w, F, gate=gate, out=[o.t for o in outs])
    for name, o in zip("qkvx", outs):
        o.check(name)


@pytest.mark.parametrize("T,odt", [(1, torch.float32), (255, torch.bfloat16), (513, torch.float32)])
def test_output_projection_writes_exactly_its_output(T, odt):
    K, N = 192, 768
    y = rnd((T, K), 42)
    w = rnd((N, K), 43, K ** -0.5)
    out = Fenced((T, N), odt)
    api.la_out_projection(y, w, out=out.t)
    out.check("out")
