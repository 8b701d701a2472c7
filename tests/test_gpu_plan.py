"""la_prefill_plan tells the truth: for each configuration the call records
timing events around exactly the kernels the plan lists (la_options_t
timing_events is the library's per-launch instrumentation hook).  Every event
is recorded once by the test before the call, then, after a short spin
kernel, a marker; an event the call re-records lies after the marker, one it
leaves alone before it (times are taken from a reference event recorded
first, so every elapsed time is positive)."""
import ctypes

import numpy as np
import pytest
import torch

from linear_attention_long_amd import _lib, inputs
from tests._util import banner

pytestmark = pytest.mark.gpu

DEV = "cuda"


class Events:
    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.arr[i] = e.value

    def record(self, i, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(self.arr[i]), ctypes.c_void_p(stream)) == 0

    def elapsed(self, a, b):
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(self.arr[b])) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.arr[a]),
                                            ctypes.c_void_p(self.arr[b])) == 0
        return ms.value

    def close(self):
        for e in self.arr:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


CASES = [
    # name, varlen, lengths (varlen) or (Bt, T), H, d, dtype, gated, normalized, chunk, out dtype
    ("fused, chunked", False, (1, 5000), 8, 128, "bf16", True, False, 0, "f32"),
    ("fused, one chunk", False, (1, 300), 8, 128, "bf16", True, False, 0, "f32"),
    ("fused, normalised, chunked", False, (2, 3001), 4, 128, "bf16", True, True, 1024, "f32"),
    ("ungated, chunked", False, (1, 5000), 8, 128, "bf16", False, False, 512, "f32"),
    ("gate not fused (H=9), bf16 out", False, (1, 700), 9, 128, "bf16", True, False, 0, "bf16"),
    ("fp32 path, d=64", False, (1, 1024), 2, 64, "f32", False, False, 128, "f32"),
    ("varlen fused, chunk on the device", True, [50, 3000, 0, 1200, 7, 2600] * 6, 8, 128, "bf16",
     True, False, 0, "f32"),
    ("varlen, one chunk each, empty sequences", True, [1, 0, 100, 64, 0, 33], 2, 128, "bf16",
     True, False, 0, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plan_matches_launches(case):
    name, varlen, shape, H, d, dt, gated, normalized, chunk, odt = case
    banner("plan vs launches: " + name)
    lib = _lib.load()
    in_dt = _lib.LA_DTYPE_BF16 if dt == "bf16" else _lib.LA_DTYPE_F32
    out_dt = _lib.LA_DTYPE_BF16 if odt == "bf16" else _lib.LA_DTYPE_F32
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    if varlen:
        lengths = shape
        cu = inputs.cu_from_lengths(lengths).to(DEV)
        nseq, total, maxlen = len(lengths), sum(lengths), max(lengths)
    else:
        nseq, T = shape
        total, maxlen = nseq * T, T
    g = torch.Generator(device=DEV).manual_seed(5)
    q, k, v = (torch.randn((total, H, d), generator=g, device=DEV).mul_(0.1).to(tdt) for _ in range(3))
    x = torch.randn((total, H * d), generator=g, device=DEV).to(tdt) if gated else None
    out = torch.empty((total, H * d), device=DEV,
                      dtype=torch.bfloat16 if odt == "bf16" else torch.float32)
    S = torch.zeros((nseq, H, d, d), device=DEV)
    z = torch.ones((nseq, H, d), device=DEV) if normalized else None
    opt = _lib.options(gated=gated, normalized=normalized, chunk_tokens=chunk)
    plan = _lib.plan(varlen, nseq, total, maxlen, H, d, in_dt, out_dt, opt)
    n = plan.n_kernels
    spare = 2
    ev = Events(2 * (n + spare) + 2)
    stream = torch.cuda.current_stream().cuda_stream
    ref, marker = 2 * (n + spare), 2 * (n + spare) + 1
    ev.record(ref, stream)
    for i in range(2 * (n + spare)):
        ev.record(i, stream)
    torch.cuda._sleep(100000)
    ev.record(marker, stream)
    opt.timing_events = ctypes.addressof(ev.arr)
    opt.n_timing = n + spare
    zp = z.data_ptr() if z is not None else None
    xp = x.data_ptr() if x is not None else None
    if varlen:
        nb = lib.la_prefill_varlen_workspace_bytes(total, nseq, maxlen, H, d, in_dt, out_dt,
                                                   ctypes.byref(opt))
        ws = torch.empty(max(int(nb), 256), dtype=torch.uint8, device=DEV)
        st = lib.la_prefill_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), xp, None,
                                   cu.data_ptr(), nseq, total, maxlen, None, zp, out.data_ptr(),
                                   S.data_ptr(), zp, H, d, in_dt, out_dt, ctypes.byref(opt),
                                   ws.data_ptr(), ws.numel(), ctypes.c_void_p(stream))
    else:
        nb = lib.la_prefill_workspace_bytes(nseq, maxlen, H, d, in_dt, out_dt, ctypes.byref(opt))
        ws = torch.empty(max(int(nb), 256), dtype=torch.uint8, device=DEV)
        st = lib.la_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), xp, None, None, zp,
                            out.data_ptr(), S.data_ptr(), zp, nseq, maxlen, H, d, in_dt, out_dt,
                            ctypes.byref(opt), ws.data_ptr(), ws.numel(), ctypes.c_void_p(stream))
    assert st == 0, _lib.load().la_status_string(st)
    torch.cuda.synchronize()
    t_marker = ev.elapsed(ref, marker)
    after = [ev.elapsed(ref, i) >= t_marker for i in range(2 * (n + spare))]
    touched = [after[2 * i] and after[2 * i + 1] for i in range(n + spare)]
    assert all(after[2 * i] == after[2 * i + 1] for i in range(n + spare)), after
    ev.close()
    print("%s: plan %s, launches timed %d" % (name, plan.kernel_names(), sum(touched)))
    assert touched == [True] * n + [False] * spare, (plan.kernel_names(), touched)
    assert np.isfinite(out.float().cpu().numpy()).all()
