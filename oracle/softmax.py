"""CPU oracle for the softmax attention layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It wraps ``sm_oracle.c`` (plain fp64
loops, built with gcc, no fast-math) and shares nothing with the HIP library.

What it computes (page title, then section):

* "六十四：MiniMax-01" (LLM tutorial, lesson 64), sections 2-3: the softmax
  layer is softmax(Q K^T / sqrt(d)) V.
* "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.2: rotary
  position embedding on half of each head's dimensions, base 10,000;
  section 4.1: base 5M, then 10M, for the long-context stages.
* "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南", section
  2.1.3: packed variable-length sequences.

The readings where the pages are silent (causal mask with the diagonal,
rotate-half pairing, grouped heads, positions restarting per sequence) are
stated in ``sm_oracle.c``.  Every function here has pins in
``tests/test_oracle_softmax_pins.py`` that do not go through the oracle's own
arithmetic (closed forms for zero keys and for two-dimensional rotations, a
library attention routine on inputs rotated by complex multiplication, the
hard-max limit, log-sum-exp).  Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sm_oracle.c")
_LIB = os.path.join(_HERE, "libsmoracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile sm_oracle.c into libsmoracle.so with gcc (-O2, no fast-math)."""
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
            lib.smo_attention.restype = ctypes.c_int
            lib.smo_attention.argtypes = [_dp, _dp, _dp, _i64p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_double, ctypes.c_double, _i64p, _i64p,
                                          ctypes.c_int64, _dp, _dp, ctypes.c_int32]
            _lib = lib
    return _lib


def _f64(a):
    """Widen any float array (numpy, or CPU torch tensor incl. bfloat16) to a
    C-contiguous float64 numpy array; the widening is exact."""
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu")
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.to(torch.float32)
        a = a.numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i64(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def attention(q, k, v, cu_seqlens=None, rotary_dim=None, rope_base=10000.0, scale=None,
              rows=None, heads=None, nthreads=None):
    """Causal softmax attention with rotary embedding, per sequence.

    q: [T, H, d]; k, v: [T, Hkv, d] (Hkv divides H); ``cu_seqlens`` [nseq + 1]
    (None: one sequence).  ``rotary_dim`` defaults to d // 2 (the pages'
    half), ``scale`` to 1/sqrt(d).  With ``rows``/``heads`` (equal-length
    index arrays) only those (token, query head) pairs are computed and
    (out [n, d], lse [n]) is returned; otherwise (out [T, H, d], lse [T, H]).
    All in fp64; lse is the natural-log log-sum-exp of the scaled scores.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, d = q.shape
    Hkv = k.shape[1]
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else _i64(cu_seqlens)
    if cu[-1] != T or k.shape != v.shape or k.shape[0] != T or k.shape[2] != d:
        raise ValueError("cu_seqlens must end at T; k and v must be [T, Hkv, d]")
    rot = d // 2 if rotary_dim is None else int(rotary_dim)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    full = rows is None
    if full:
        rows = np.repeat(np.arange(T, dtype=np.int64), H)
        heads = np.tile(np.arange(H, dtype=np.int64), T)
    rows, heads = _i64(rows), _i64(heads)
    n = len(rows)
    out = np.zeros((n, d))
    lse = np.zeros(n)
    nt = int(nthreads) if nthreads else max(1, os.cpu_count() or 1)
    rc = lib.smo_attention(q.ctypes.data_as(_dp), k.ctypes.data_as(_dp), v.ctypes.data_as(_dp),
                           cu.ctypes.data_as(_i64p), len(cu) - 1, H, Hkv, d, rot,
                           float(rope_base), sc, rows.ctypes.data_as(_i64p),
                           heads.ctypes.data_as(_i64p), n, out.ctypes.data_as(_dp),
                           lse.ctypes.data_as(_dp), nt)
    if rc != 0:
        raise ValueError("smo_attention rejected its arguments")
    if full:
        return out.reshape(T, H, d), lse.reshape(T, H)
    return out, lse
