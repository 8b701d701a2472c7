"""CPU oracle for causal linear attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It wraps ``la_oracle.c`` (plain fp64
loops, built with gcc, no fast-math) and shares nothing with the HIP library.

What it computes follows the pages (page title, then section):

* "六十四：MiniMax-01" (LLM tutorial, lesson 64), section 3 "Lightning
  Attention 的定位": the causal sum over i <= t, the recurrent state
  S_t = S_{t-1} + phi(k_t) v_t^T and normaliser z_t = z_{t-1} + phi(k_t);
  the optional normalised output divides phi(q_t)^T S_t by phi(q_t)^T z_t.
* "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1: SiLU on Q, K
  and V; output RMSNorm(Y) * sigmoid(X).

Every function here has pins that do not go through the oracle's own formula:
``tests/test_oracle_pins.py`` (brute-force masked quadratic form, closed
forms for constant inputs, T = 1, the non-causal last row, state chaining,
decode = prefill, varlen = per sequence, block-size invariance, gate
invariants), ``tests/test_oracle_featurized_pins.py`` (inputs given as
features) and ``tests/test_oracle_sampled_f32_pins.py`` (the float-input
sampled form: bit-for-bit equal to the fp64 recurrence and equal to the
masked quadratic form across sequence boundaries, empty sequences, duplicate
samples and carried states).  Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp32 = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile la_oracle.c into liblaoracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
               "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            lib.lao_prefill.restype = ctypes.c_int
            lib.lao_prefill.argtypes = [_dp, _dp, _dp, _i64p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, _dp, _dp, ctypes.c_int32, _dp, _dp, _dp,
                                        _i64p, ctypes.c_int64, ctypes.c_int32]
            lib.lao_prefill_f32in.restype = ctypes.c_int
            lib.lao_prefill_f32in.argtypes = [_fp32, _fp32, _fp32, _i64p, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, _dp, _dp,
                                              ctypes.c_int32, _dp, _dp, _dp, _i64p, ctypes.c_int64,
                                              ctypes.c_int32]
            lib.lao_prefill_blocked.restype = ctypes.c_int
            lib.lao_prefill_blocked.argtypes = [_dp, _dp, _dp, _i64p, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, _dp, _dp,
                                                ctypes.c_int32, _dp, _dp, _dp, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32]
            lib.lao_decode_step.restype = ctypes.c_int
            lib.lao_decode_step.argtypes = [_dp, _dp, _dp, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, _dp, _dp, _dp]
            lib.lao_gate.restype = ctypes.c_int
            lib.lao_gate.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_double, _dp]
            _lib = lib
    return _lib


def _f64(a):
    """Widen any float array (numpy, or CPU torch tensor incl. bfloat16) to a
    C-contiguous float64 numpy array; the widening is exact."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        import torch

        a = a.detach().to("cpu")
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.to(torch.float32)
        a = a.numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _nthreads(n):
    return int(n) if n else max(1, os.cpu_count() or 1)


def _flags(normalized, featurized):
    """The C oracle's flags word: bit 0 normalised output, bit 1 the inputs
    are already feature vectors (the feature map is not applied again)."""
    return (1 if normalized else 0) | (2 if featurized else 0)


def _cu_array(cu_seqlens, total):
    if cu_seqlens is None:
        return np.array([0, total], dtype=np.int64)
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def prefill(q, k, v, cu_seqlens=None, state_in=None, z_in=None, normalized=False,
            featurized=False, sample_idx=None, nthreads=None):
    """Recurrent form, token by token, of the causal linear attention.

    q, k, v: [total_T, H, d] pre-activation values (a single sequence when
    ``cu_seqlens`` is None).  Returns (y, state_out, z_out) in fp64: y is
    [total_T, H, d], or [len(sample_idx), H, d] when ``sample_idx`` (sorted
    global token indices) is given; state_out [nseq, H, d, d]; z_out
    [nseq, H, d] (zeros unless normalized or z_in given).  With
    ``featurized`` q, k, v are taken as feature vectors phi(.) already (the
    feature map was applied where they were produced) and used as given.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    total, H, d = q.shape
    cu = _cu_array(cu_seqlens, total)
    nseq = len(cu) - 1
    si = _f64(state_in)
    zi = _f64(z_in)
    if sample_idx is not None:
        sample_idx = np.ascontiguousarray(np.asarray(sample_idx, dtype=np.int64))
        y = np.zeros((len(sample_idx), H, d))
    else:
        y = np.zeros((total, H, d))
    so = np.zeros((nseq, H, d, d))
    zo = np.zeros((nseq, H, d))
    rc = lib.lao_prefill(_ptr(q), _ptr(k), _ptr(v), cu.ctypes.data_as(_i64p), nseq, H, d,
                         _ptr(si), _ptr(zi), _flags(normalized, featurized), _ptr(y), _ptr(so), _ptr(zo),
                         None if sample_idx is None else sample_idx.ctypes.data_as(_i64p),
                         0 if sample_idx is None else len(sample_idx), _nthreads(nthreads))
    if rc != 0:
        raise ValueError("lao_prefill rejected its arguments")
    return y, so, zo


def prefill_blocked(q, k, v, block, cu_seqlens=None, state_in=None, z_in=None,
                    normalized=False, featurized=False, fp32=False, nthreads=None):
    """Blocked form (masked quadratic within blocks of ``block`` tokens, the
    carried state across blocks), in fp64 or fp32 arithmetic.  Same returns as
    :func:`prefill`.  Used to check block-size invariance."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    total, H, d = q.shape
    cu = _cu_array(cu_seqlens, total)
    nseq = len(cu) - 1
    y = np.zeros((total, H, d))
    so = np.zeros((nseq, H, d, d))
    zo = np.zeros((nseq, H, d))
    rc = lib.lao_prefill_blocked(_ptr(q), _ptr(k), _ptr(v), cu.ctypes.data_as(_i64p), nseq, H, d,
                                 _ptr(_f64(state_in)), _ptr(_f64(z_in)), _flags(normalized, featurized),
                                 _ptr(y), _ptr(so), _ptr(zo), int(block), int(bool(fp32)),
                                 _nthreads(nthreads))
    if rc != 0:
        raise ValueError("lao_prefill_blocked rejected its arguments")
    return y, so, zo


def decode_step(q, k, v, S, z=None, normalized=False, featurized=False):
    """One decode token per sequence.  q, k, v: [N, H, d]; S: [N, H, d, d];
    z: [N, H, d].  Returns (y, S_new, z_new); the inputs are not modified."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, H, d = q.shape
    S = _f64(S).copy()
    z = np.zeros((N, H, d)) if z is None else _f64(z).copy()
    y = np.zeros((N, H, d))
    rc = lib.lao_decode_step(_ptr(q), _ptr(k), _ptr(v), N, H, d, _flags(normalized, featurized),
                             _ptr(S), _ptr(z), _ptr(y))
    if rc != 0:
        raise ValueError("lao_decode_step rejected its arguments")
    return y, S, z


def gate(y, x, w=None, group=0, eps=1e-6):
    """RMSNorm(y) * w * sigmoid(x) per token.  y, x: [ntok, F] (any leading
    shape is flattened to tokens x features); group 0 = all F features."""
    lib = _load()
    y = _f64(y)
    x = _f64(x)
    shape = y.shape
    F = shape[-1]
    y2 = np.ascontiguousarray(y.reshape(-1, F))
    x2 = np.ascontiguousarray(x.reshape(-1, F))
    w2 = None if w is None else np.ascontiguousarray(_f64(w).reshape(F))
    out = np.zeros_like(y2)
    rc = lib.lao_gate(_ptr(y2), _ptr(x2), _ptr(w2), y2.shape[0], F, int(group) if group else F,
                      float(eps), _ptr(out))
    if rc != 0:
        raise ValueError("lao_gate rejected its arguments")
    return out.reshape(shape)


def forward(q, k, v, x=None, w=None, cu_seqlens=None, state_in=None, z_in=None,
            normalized=False, featurized=False, gated=False, norm_group=0, eps=1e-6, nthreads=None):
    """Whole path: recurrence, then (if gated) the RMSNorm * sigmoid gate.
    Returns (out [total_T, H*d], state_out, z_out) in fp64."""
    y, so, zo = prefill(q, k, v, cu_seqlens, state_in, z_in, normalized, featurized,
                        nthreads=nthreads)
    total, H, d = y.shape
    y = y.reshape(total, H * d)
    if gated:
        y = gate(y, _f64(x).reshape(total, H * d), w, norm_group, eps)
    return y, so, zo


def _f32(a):
    """Float inputs as a C-contiguous float32 numpy array (bf16 widens exactly)."""
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu")
        if a.dtype != torch.float32:
            a = a.to(torch.float32)
        return np.ascontiguousarray(a.numpy())
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def prefill_sampled_f32(q, k, v, sample_idx, cu_seqlens=None, state_in=None, z_in=None,
                        normalized=False, featurized=False, nthreads=None):
    """:func:`prefill` at the listed tokens for float32-valued inputs (bf16 or
    fp32 values), widened to double one token at a time inside the oracle."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    total, H, d = q.shape
    cu = _cu_array(cu_seqlens, total)
    nseq = len(cu) - 1
    sample_idx = np.ascontiguousarray(np.asarray(sample_idx, dtype=np.int64))
    y = np.zeros((len(sample_idx), H, d))
    so = np.zeros((nseq, H, d, d))
    zo = np.zeros((nseq, H, d))
    fp = lambda a: a.ctypes.data_as(_fp32)
    rc = lib.lao_prefill_f32in(fp(q), fp(k), fp(v), cu.ctypes.data_as(_i64p), nseq, H, d,
                               _ptr(_f64(state_in)), _ptr(_f64(z_in)), _flags(normalized, featurized),
                               _ptr(y), _ptr(so), _ptr(zo), sample_idx.ctypes.data_as(_i64p),
                               len(sample_idx), _nthreads(nthreads))
    if rc != 0:
        raise ValueError("lao_prefill_f32in rejected its arguments")
    return y, so, zo


def forward_sampled(q, k, v, sample_idx, x=None, w=None, cu_seqlens=None, state_in=None,
                    z_in=None, normalized=False, featurized=False, gated=False, norm_group=0, eps=1e-6,
                    nthreads=None):
    """The path's output only at the listed tokens (sorted global indices),
    for inputs too long to hold every fp64 output.  Returns (out [n, H*d],
    state_out, z_out)."""
    sample_idx = np.asarray(sample_idx, dtype=np.int64)
    y, so, zo = prefill(q, k, v, cu_seqlens, state_in, z_in, normalized, featurized,
                        sample_idx=sample_idx, nthreads=nthreads)
    n, H, d = y.shape
    y = y.reshape(n, H * d)
    if gated:
        xs = _f64(x[sample_idx] if not hasattr(x, "detach") else x[sample_idx.tolist()])
        y = gate(y, xs.reshape(n, H * d), w, norm_group, eps)
    return y, so, zo
