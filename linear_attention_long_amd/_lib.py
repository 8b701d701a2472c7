"""ctypes view of liblinattn.so (the C ABI declared in include/la.h,
include/la_softmax.h and include/la_proj.h)."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinattn.so")

LA_OK = 0
LA_ERR_INVALID_ARGUMENT = 1
LA_ERR_UNSUPPORTED = 2
LA_ERR_WORKSPACE_TOO_SMALL = 3
LA_ERR_HIP = 4
LA_ERR_WAIT_TIMEOUT = 5

LA_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/la.h

LA_DTYPE_F32 = 0
LA_DTYPE_BF16 = 1

# every extern "C" function declared in include/la.h, include/la_softmax.h and
# include/la_proj.h
EXPORTS = (
    "la_default_options",
    "la_prefill",
    "la_prefill_noalloc",
    "la_prefill_varlen",
    "la_decode_step",
    "la_prefill_workspace_bytes",
    "la_prefill_varlen_workspace_bytes",
    "la_decode_workspace_bytes",
    "la_prefill_plan",
    "la_prefill_wait_status",
    "la_schedule_step",
    "la_serve_step",
    "la_serve_step_workspace_bytes",
    "la_status_string",
    "la_softmax_default_options",
    "la_softmax_attention_varlen",
    "la_softmax_workspace_bytes",
    "la_proj_default_options",
    "la_qkvx_projection",
    "la_out_projection",
)


class Options(ctypes.Structure):
    _fields_ = [
        ("block_size", ctypes.c_int32),
        ("normalized", ctypes.c_int32),
        ("gated", ctypes.c_int32),
        ("norm_group", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("chunk_tokens", ctypes.c_int32),
        ("timing_events", ctypes.c_void_p),
        ("n_timing", ctypes.c_int32),
        ("state_slots", ctypes.c_void_p),
        ("state_rows", ctypes.c_int32),
        ("featurized", ctypes.c_int32),
        ("wait_spin_limit", ctypes.c_int32),
        ("state_access", ctypes.c_int32),
    ]


# la_kernel_t: kernels of a prefill call, as listed by la_prefill_plan
KERNEL_NAMES = {
    1: "chunk_table",
    2: "state_copy",
    3: "chunk_state",
    4: "chunk_scan",
    5: "exchange_clear",
    6: "main",
    7: "main_gated",
    8: "gate",
}


class SoftmaxOptions(ctypes.Structure):
    _fields_ = [
        ("rotary_dim", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("scale", ctypes.c_float),
        ("timing_events", ctypes.c_void_p),
        ("n_timing", ctypes.c_int32),
        ("precision", ctypes.c_int32),
    ]


class ProjOptions(ctypes.Structure):
    _fields_ = [
        ("featurize", ctypes.c_int32),
        ("timing_events", ctypes.c_void_p),
        ("n_timing", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("main_workgroups", ctypes.c_int64),
        ("chunk_tokens", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("fused_gate", ctypes.c_int32),
        ("chunk_on_device", ctypes.c_int32),
        ("n_kernels", ctypes.c_int32),
        ("kernels", ctypes.c_int32 * 8),
        ("status_offset", ctypes.c_int64),
    ]

    def kernel_names(self):
        return [KERNEL_NAMES[self.kernels[i]] for i in range(self.n_kernels)]


class Request(ctypes.Structure):
    _fields_ = [("remaining", ctypes.c_int32), ("slot", ctypes.c_int32)]


class Step(ctypes.Structure):
    _fields_ = [
        ("num_decode", ctypes.c_int32),
        ("num_prefill", ctypes.c_int32),
        ("prefill_tokens", ctypes.c_int32),
        ("max_chunk", ctypes.c_int32),
    ]


class LAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_fp = ctypes.c_void_p  # float* passed as raw addresses
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_optp = ctypes.POINTER(Options)


def load() -> ctypes.CDLL:
    """Load liblinattn.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liblinattn.so is not built (expected at %s); run "
                               "`python -m linear_attention_long_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        lib.la_default_options.restype = Options
        lib.la_default_options.argtypes = []
        lib.la_status_string.restype = ctypes.c_char_p
        lib.la_status_string.argtypes = [ctypes.c_int]
        lib.la_prefill.restype = ctypes.c_int
        lib.la_prefill.argtypes = [_vp, _vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp, _fp,
                                   _i32, _i32, _i32, _i32, ctypes.c_int, ctypes.c_int,
                                   _optp, _vp, _sz, _vp]
        lib.la_prefill_noalloc.restype = ctypes.c_int
        lib.la_prefill_noalloc.argtypes = [_vp, _vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp, _fp,
                                           _i32, _i32, _i32, _i32, ctypes.c_int, ctypes.c_int,
                                           _optp, _vp]
        lib.la_prefill_varlen.restype = ctypes.c_int
        lib.la_prefill_varlen.argtypes = [_vp, _vp, _vp, _vp, _fp, _vp, _i32, _i32, _i32,
                                          _fp, _fp, _vp, _fp, _fp, _i32, _i32, ctypes.c_int,
                                          ctypes.c_int, _optp, _vp, _sz, _vp]
        lib.la_decode_step.restype = ctypes.c_int
        lib.la_decode_step.argtypes = [_vp, _vp, _vp, _vp, _fp, _fp, _fp, _vp, _i32, _i32, _i32,
                                       ctypes.c_int, ctypes.c_int, _optp, _vp, _sz, _vp]
        lib.la_prefill_workspace_bytes.restype = _sz
        lib.la_prefill_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, ctypes.c_int,
                                                   ctypes.c_int, _optp]
        lib.la_prefill_varlen_workspace_bytes.restype = _sz
        lib.la_prefill_varlen_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32,
                                                          ctypes.c_int, ctypes.c_int, _optp]
        lib.la_decode_workspace_bytes.restype = _sz
        lib.la_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, ctypes.c_int, _optp]
        lib.la_prefill_plan.restype = ctypes.c_int
        lib.la_prefill_plan.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                        ctypes.c_int, _i32, _optp, ctypes.POINTER(Plan)]
        lib.la_prefill_wait_status.restype = ctypes.c_int
        lib.la_prefill_wait_status.argtypes = [_vp, ctypes.c_int64, _vp]
        lib.la_schedule_step.restype = ctypes.c_int
        lib.la_schedule_step.argtypes = [ctypes.POINTER(Request), _i32, _i32,
                                         ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                         ctypes.POINTER(Step)]
        lib.la_serve_step.restype = ctypes.c_int
        lib.la_serve_step.argtypes = [_vp, _vp, _vp, _vp, _fp, _fp, _fp, _i32, _vp, _i32, _vp, _vp,
                                      _i32, _i32, _i32, _vp, _i32, _i32, ctypes.c_int,
                                      ctypes.c_int, _optp, _vp, _sz, _vp, _vp]
        lib.la_serve_step_workspace_bytes.restype = _sz
        lib.la_serve_step_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32,
                                                      ctypes.c_int, ctypes.c_int, _optp]
        lib.la_softmax_default_options.restype = SoftmaxOptions
        lib.la_softmax_default_options.argtypes = []
        lib.la_softmax_attention_varlen.restype = ctypes.c_int
        lib.la_softmax_attention_varlen.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                    _i32, _i32, ctypes.c_int, ctypes.c_int, _vp,
                                                    _fp, ctypes.POINTER(SoftmaxOptions), _vp, _sz,
                                                    _vp]
        lib.la_softmax_workspace_bytes.restype = _sz
        lib.la_softmax_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32,
                                                   ctypes.c_int, ctypes.c_int,
                                                   ctypes.POINTER(SoftmaxOptions)]
        lib.la_proj_default_options.restype = ProjOptions
        lib.la_proj_default_options.argtypes = []
        lib.la_qkvx_projection.restype = ctypes.c_int
        lib.la_qkvx_projection.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                           ctypes.c_int, ctypes.POINTER(ProjOptions), _vp]
        lib.la_out_projection.restype = ctypes.c_int
        lib.la_out_projection.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, ctypes.c_int,
                                          ctypes.POINTER(ProjOptions), _vp]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load().la_status_string(int(status)).decode()
    except Exception:  # library missing: still give a message
        return "status %d" % status


def options(block_size=0, normalized=False, gated=False, norm_group=0, rms_eps=1e-6,
            chunk_tokens=0, featurized=False, wait_spin_limit=0, state_access=0) -> Options:
    o = load().la_default_options()
    o.block_size = int(block_size)
    o.normalized = int(bool(normalized))
    o.gated = int(bool(gated))
    o.norm_group = int(norm_group)
    o.rms_eps = float(rms_eps)
    o.chunk_tokens = int(chunk_tokens)
    o.featurized = int(bool(featurized))
    o.wait_spin_limit = int(wait_spin_limit)
    o.state_access = int(state_access)
    return o


def softmax_options(rotary_dim=-1, rope_base=10000.0, scale=0.0, precision=1) -> SoftmaxOptions:
    o = load().la_softmax_default_options()
    o.rotary_dim = int(rotary_dim)
    o.rope_base = float(rope_base)
    o.scale = float(scale)
    o.precision = int(precision)
    return o


def proj_options(featurize=True) -> ProjOptions:
    o = load().la_proj_default_options()
    o.featurize = int(bool(featurize))
    return o


def plan(varlen, num_seqs, total_T, max_seqlen, H, d, in_dtype, out_dtype, opt,
         has_state_out=True) -> Plan:
    """What a prefill call with these sizes will launch (la_prefill_plan)."""
    r = Plan()
    check(load().la_prefill_plan(int(bool(varlen)), num_seqs, total_T, max_seqlen, H, d,
                                 in_dtype, out_dtype, int(bool(has_state_out)),
                                 ctypes.byref(opt), ctypes.byref(r)), "la_prefill_plan")
    return r


def check(status: int, where: str) -> None:
    if status != LA_OK:
        raise LAError(status, where)
