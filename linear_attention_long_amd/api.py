"""Python entry points with the names of the C ABI: argument marshalling only.

Every step of the computation runs in liblinattn's HIP kernels; torch supplies
device memory (outputs and workspace) and the current stream.  If the library
is not built, every call raises.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DT = {torch.float32: _lib.LA_DTYPE_F32, torch.bfloat16: _lib.LA_DTYPE_BF16}


def _dtype(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError("dtype %s not supported (float32 or bfloat16)" % t)
    return _DT[t]


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _bf16(t, name):
    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16 (got %s)" % (name, t.dtype))
    return t


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, given=None) -> torch.Tensor | None:
    if nbytes == ctypes.c_size_t(-1).value:
        return None
    if nbytes == 0:
        return None
    if given is not None:
        if given.dtype != torch.uint8 or given.numel() < nbytes:
            raise ValueError("workspace must be a uint8 tensor of at least %d bytes" % nbytes)
        return given
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def _keep_for(stream, *tensors):
    """Buffers allocated here on the current stream but used by kernels on
    ``stream``: tell the caching allocator, so that it does not hand their
    memory to another allocation before that stream's work is done."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def la_prefill(q, k, v, x=None, w=None, state_in=None, z_in=None, *, normalized=False,
               block_size=0, norm_group=0, rms_eps=1e-6, chunk_tokens=0,
               out_dtype=torch.float32, return_state=True, featurized=False, stream=None,
               workspace=None, wait_spin_limit=0):
    """Prefill of Bt equal-length sequences.

    q, k, v: [Bt, T, H, d] (or [T, H, d]) pre-activation, float32 or bfloat16.
    x: gate pre-activation [Bt, T, H*d] (same dtype) -> gated output, or None.
    w: RMSNorm weight [H*d] float32 or None.  state_in [Bt, H, d, d], z_in
    [Bt, H, d] float32 or None.  Returns (out [Bt, T, H*d], state_out, z_out).
    ``featurized``: q, k, v are feature vectors already (SiLU applied where
    they were produced).  ``workspace``: a uint8 device tensor to use as the
    call's workspace (else one is allocated); pass one to read the call's
    wait status afterwards (:func:`la_prefill_wait_status`).
    ``wait_spin_limit``: bound of the fused gate's waits (0 = default).
    """
    lib = _lib.load()
    squeeze = q.dim() == 3
    if squeeze:
        q, k, v = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
        if x is not None:
            x = x.unsqueeze(0)
        if state_in is not None and state_in.dim() == 3:
            state_in = state_in.unsqueeze(0)
        if z_in is not None and z_in.dim() == 2:
            z_in = z_in.unsqueeze(0)
    Bt, T, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same shape and dtype")
    gated = x is not None
    opt = _lib.options(block_size, normalized, gated, norm_group, rms_eps, chunk_tokens,
                       featurized, wait_spin_limit)
    in_dt, out_dt = _dtype(q.dtype), _dtype(out_dtype)
    dev = q.device
    out = torch.empty((Bt, T, H * d), dtype=out_dtype, device=dev)
    state_out = torch.empty((Bt, H, d, d), dtype=torch.float32, device=dev) if return_state else None
    z_out = (torch.empty((Bt, H, d), dtype=torch.float32, device=dev)
             if (return_state and normalized) else None)
    nbytes = lib.la_prefill_workspace_bytes(Bt, T, H, d, in_dt, out_dt, ctypes.byref(opt))
    ws = _workspace(nbytes, dev, workspace)
    st = lib.la_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(w), _ptr(state_in), _ptr(z_in),
                        _ptr(out), _ptr(state_out), _ptr(z_out), Bt, T, H, d, in_dt, out_dt,
                        ctypes.byref(opt), _ptr(ws), 0 if ws is None else ws.numel(),
                        _stream(stream))
    _lib.check(st, "la_prefill")
    _keep_for(stream, out, state_out, z_out, ws)
    if squeeze:
        out = out[0]
        state_out = None if state_out is None else state_out[0]
        z_out = None if z_out is None else z_out[0]
    return out, state_out, z_out


def _slots(opt, state_slots, pool):
    """Slot table (int32 on the GPU) over a state pool [rows, H, d, d]."""
    if state_slots is None:
        return None
    if state_slots.dtype != torch.int32:
        raise TypeError("state_slots must be int32")
    if pool is None:
        raise ValueError("state_slots needs the state pool")
    opt.state_slots = _ptr(state_slots).value
    opt.state_rows = int(pool.shape[0])
    return state_slots


def la_prefill_varlen(q, k, v, cu_seqlens, max_seqlen, x=None, w=None, state_in=None, z_in=None,
                      *, normalized=False, block_size=0, norm_group=0, rms_eps=1e-6,
                      chunk_tokens=0, out_dtype=torch.float32, return_state=True,
                      state_slots=None, out=None, featurized=False, stream=None,
                      workspace=None, wait_spin_limit=0):
    """Prefill of a packed batch.  q, k, v: [total_T, H, d]; cu_seqlens: int32
    [num_seqs + 1] on the GPU; max_seqlen: host int bounding every length.
    Returns (out [total_T, H*d], state_out [num_seqs, H, d, d], z_out).
    With ``state_slots`` (int32 [num_seqs] on the GPU), state_in / z_in are
    pools of per-request states indexed by slot and are updated in place;
    they are returned as the states."""
    lib = _lib.load()
    total_T, H, d = q.shape
    num_seqs = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    gated = x is not None
    opt = _lib.options(block_size, normalized, gated, norm_group, rms_eps, chunk_tokens,
                       featurized, wait_spin_limit)
    _slots(opt, state_slots, state_in)
    in_dt, out_dt = _dtype(q.dtype), _dtype(out_dtype)
    dev = q.device
    if out is None:
        out = torch.empty((total_T, H * d), dtype=out_dtype, device=dev)
    if state_slots is not None:
        state_out, z_out = state_in, z_in
    else:
        state_out = (torch.empty((num_seqs, H, d, d), dtype=torch.float32, device=dev)
                     if return_state else None)
        z_out = (torch.empty((num_seqs, H, d), dtype=torch.float32, device=dev)
                 if (return_state and normalized) else None)
    nbytes = lib.la_prefill_varlen_workspace_bytes(total_T, num_seqs, int(max_seqlen), H, d,
                                                   in_dt, out_dt, ctypes.byref(opt))
    ws = _workspace(nbytes, dev, workspace)
    st = lib.la_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(w), _ptr(cu_seqlens),
                               num_seqs, total_T, int(max_seqlen), _ptr(state_in), _ptr(z_in),
                               _ptr(out), _ptr(state_out), _ptr(z_out), H, d, in_dt, out_dt,
                               ctypes.byref(opt), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream(stream))
    _lib.check(st, "la_prefill_varlen")
    _keep_for(stream, out, state_out, z_out, ws)
    return out, state_out, z_out


def la_prefill_wait_status(workspace, status_offset, stream=None) -> int:
    """Status of the bounded waits of a finished prefill call
    (la_prefill_wait_status): synchronises ``stream`` and reads the word at
    ``status_offset`` (la_plan_t.status_offset of the call's plan) of the
    call's ``workspace``.  Returns LA_OK (0) or LA_ERR_WAIT_TIMEOUT (5)."""
    lib = _lib.load()
    st = lib.la_prefill_wait_status(_ptr(workspace), int(status_offset), _stream(stream))
    if st not in (_lib.LA_OK, _lib.LA_ERR_WAIT_TIMEOUT):
        _lib.check(st, "la_prefill_wait_status")
    return st



def la_decode_step(q, k, v, state, z=None, x=None, w=None, *, normalized=False, norm_group=0,
                   rms_eps=1e-6, out_dtype=torch.float32, out=None, workspace=None,
                   state_slots=None, featurized=False, stream=None, state_access=0):
    """One decode token per sequence.  q, k, v: [N, H, d]; state [N, H, d, d]
    float32 and z [N, H, d] (normalised mode) are updated in place (with
    ``state_slots``, int32 [N] on the GPU: pools [rows, H, d, d] / [rows, H, d]
    indexed by slot).  Returns out [N, H*d].  ``out``/``workspace`` may be
    passed to reuse buffers.  ``state_access``: 0 auto, 1 streaming
    (non-temporal), 2 cache-resident (include/la.h); results are identical."""
    lib = _lib.load()
    N, H, d = q.shape
    gated = x is not None
    opt = _lib.options(64, normalized, gated, norm_group, rms_eps, 0, featurized,
                       state_access=state_access)
    _slots(opt, state_slots, state)
    in_dt, out_dt = _dtype(q.dtype), _dtype(out_dtype)
    if out is None:
        out = torch.empty((N, H * d), dtype=out_dtype, device=q.device)
    if workspace is None:
        nbytes = lib.la_decode_workspace_bytes(N, H, d, out_dt, ctypes.byref(opt))
        workspace = _workspace(nbytes, q.device)
    st = lib.la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(w), _ptr(state), _ptr(z),
                            _ptr(out), N, H, d, in_dt, out_dt, ctypes.byref(opt),
                            _ptr(workspace), 0 if workspace is None else workspace.numel(),
                            _stream(stream))
    _lib.check(st, "la_decode_step")
    _keep_for(stream, out, workspace)
    return out


def la_schedule_step(remaining, max_batched_tokens=32768):
    """Host-side step choice (la_schedule_step) for requests with the given
    remaining prompt tokens (0 = decoding).  Returns (order, chunk, step):
    packed sequence i of the step is request order[i] with chunk[i] tokens;
    step has num_decode, num_prefill, prefill_tokens, max_chunk."""
    lib = _lib.load()
    R = len(remaining)
    reqs = (_lib.Request * max(R, 1))()
    for i, r in enumerate(remaining):
        reqs[i].remaining = int(r)
        reqs[i].slot = i
    order = (ctypes.c_int32 * max(R, 1))()
    chunk = (ctypes.c_int32 * max(R, 1))()
    step = _lib.Step()
    _lib.check(lib.la_schedule_step(reqs, R, int(max_batched_tokens), order, chunk,
                                    ctypes.byref(step)), "la_schedule_step")
    n = step.num_decode + step.num_prefill
    return list(order)[:n], list(chunk)[:n], step


def la_serve_step(q, k, v, state_pool, decode_slots, prefill_cu, prefill_slots, max_chunk,
                  x=None, w=None, z_pool=None, *, normalized=False, norm_group=0, rms_eps=1e-6,
                  out_dtype=torch.float32, out=None, decode_stream=None, prefill_stream=None,
                  featurized=False):
    """One serving step (la_serve_step): rows [0, len(decode_slots)) of the
    packed q, k, v (and x) are decode tokens, the rest prefill chunks at
    prefill_cu (int32 on the GPU, relative offsets); decode_slots and
    prefill_slots (int32 on the GPU) index the state pool, updated in place.
    The two parts are enqueued on decode_stream and prefill_stream."""
    lib = _lib.load()
    rows, H, d = q.shape
    nd = decode_slots.numel() if decode_slots is not None else 0
    npf = prefill_slots.numel() if prefill_slots is not None else 0
    ptok = rows - nd
    opt = _lib.options(0, normalized, x is not None, norm_group, rms_eps, 0, featurized)
    in_dt, out_dt = _dtype(q.dtype), _dtype(out_dtype)
    if out is None:
        out = torch.empty((rows, H * d), dtype=out_dtype, device=q.device)
    nbytes = lib.la_serve_step_workspace_bytes(nd, npf, ptok, int(max_chunk), H, d, in_dt, out_dt,
                                               ctypes.byref(opt))
    ws = _workspace(nbytes, q.device)
    st = lib.la_serve_step(_ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(w), _ptr(state_pool),
                           _ptr(z_pool), int(state_pool.shape[0]),
                           _ptr(decode_slots) if nd else None, nd,
                           _ptr(prefill_cu) if npf else None, _ptr(prefill_slots) if npf else None,
                           npf, ptok, int(max_chunk), _ptr(out), H, d, in_dt, out_dt,
                           ctypes.byref(opt), _ptr(ws), 0 if ws is None else ws.numel(),
                           _stream(decode_stream), _stream(prefill_stream))
    _lib.check(st, "la_serve_step")
    # the buffers made here are used on the two streams: keep the caching
    # allocator from reusing them before that work is done
    for t in (out, ws):
        if t is not None:
            for sm in (decode_stream, prefill_stream):
                if sm is not None:
                    t.record_stream(sm)
    return out


# the same calls under short names
prefill = la_prefill
prefill_varlen = la_prefill_varlen
decode_step = la_decode_step
schedule_step = la_schedule_step
serve_step = la_serve_step


def la_softmax_attention_varlen(q, k, v, cu_seqlens, max_seqlen, *, rotary_dim=-1,
                                rope_base=10000.0, scale=0.0, precision=1,
                                out_dtype=torch.bfloat16, return_lse=False, out=None,
                                stream=None):
    """Causal softmax attention with rotary embedding over a packed batch
    (the hybrid model's softmax layer).  q: [total_T, H, d] bfloat16; k, v:
    [total_T, H_kv, d] bfloat16 (H_kv divides H); cu_seqlens: int32
    [num_seqs + 1] on the GPU; max_seqlen: host int bounding every length.
    rotary_dim -1 = d/2; scale 0 = 1/sqrt(d); precision 1 (default) = split
    (hi + lo) operands in both products, within 1e-2 of the output's rms;
    2 = fp16 operands, one product each (faster; within that bound for
    scores of unit spread, error growing with the spread); 0 = single bf16
    operands (fastest, loosest).  Returns (out [total_T, H, d],
    lse [total_T, H] float32 or None)."""
    lib = _lib.load()
    total_T, H, d = q.shape
    H_kv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != total_T or k.shape[2] != d:
        raise ValueError("k and v must be [total_T, H_kv, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same dtype")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    num_seqs = cu_seqlens.numel() - 1
    opt = _lib.softmax_options(rotary_dim, rope_base, scale, precision)
    in_dt, out_dt = _dtype(q.dtype), _dtype(out_dtype)
    dev = q.device
    if out is None:
        out = torch.empty((total_T, H, d), dtype=out_dtype, device=dev)
    lse = torch.empty((total_T, H), dtype=torch.float32, device=dev) if return_lse else None
    nbytes = lib.la_softmax_workspace_bytes(num_seqs, total_T, int(max_seqlen), H, H_kv, d,
                                            in_dt, out_dt, ctypes.byref(opt))
    ws = _workspace(nbytes, dev)
    st = lib.la_softmax_attention_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), num_seqs,
                                         total_T, int(max_seqlen), H, H_kv, d, in_dt, out_dt,
                                         _ptr(out), _ptr(lse), ctypes.byref(opt), _ptr(ws),
                                         0 if ws is None else ws.numel(), _stream(stream))
    _lib.check(st, "la_softmax_attention_varlen")
    _keep_for(stream, out, lse, ws)
    return out, lse


def la_qkvx_projection(hidden, weight, F, *, gate=True, featurize=True, out_dtype=torch.bfloat16,
                       out=None, stream=None):
    """The layer's input projection (include/la_proj.h): hidden [T, K] bf16,
    weight [nblk * F, K] bf16 with rows [W_q; W_k; W_v; W_g] (nblk = 4 with
    ``gate``, else 3).  Returns (q, k, v, x_gate), each [T, F] ``out_dtype``
    (x_gate None without ``gate``); q, k, v carry SiLU when ``featurize``.
    ``out``: four (or three) preallocated outputs to write instead."""
    lib = _lib.load()
    _bf16(hidden, "hidden")
    _bf16(weight, "weight")
    T, K = hidden.shape
    nblk = 4 if gate else 3
    if weight.shape != (nblk * F, K):
        raise ValueError("weight must be [%d * F, K]" % nblk)
    if out is None:
        out = [torch.empty((T, F), dtype=out_dtype, device=hidden.device) for _ in range(nblk)]
    if len(out) != nblk or any(o.shape != (T, F) or o.dtype != out[0].dtype for o in out):
        raise ValueError("out must be %d tensors [T, F] of one dtype" % nblk)
    out_dtype = out[0].dtype
    outs = list(out) + [None] * (4 - len(out))
    opt = _lib.proj_options(featurize)
    st = lib.la_qkvx_projection(_ptr(hidden), _ptr(weight), _ptr(outs[0]), _ptr(outs[1]),
                                _ptr(outs[2]), _ptr(outs[3]), T, K, F, _dtype(out_dtype),
                                ctypes.byref(opt), _stream(stream))
    _lib.check(st, "la_qkvx_projection")
    _keep_for(stream, *outs)
    return tuple(outs)


def la_out_projection(y, weight, *, out_dtype=torch.bfloat16, out=None, stream=None):
    """The layer's output projection (include/la_proj.h): y [T, K] bf16 (the
    gated attention output of these heads, K = H * d), weight [N, K] bf16
    (the O projection's columns for these heads, row n = hidden feature n).
    Returns y @ weight^T, [T, N] ``out_dtype``: this device's partial sum of
    the layer output.  ``out``: a preallocated [T, N] output to write instead."""
    lib = _lib.load()
    _bf16(y, "y")
    _bf16(weight, "weight")
    T, K = y.shape
    N, Kw = weight.shape
    if Kw != K:
        raise ValueError("weight must be [N, K] with K = y's width")
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype, device=y.device)
    if out.shape != (T, N):
        raise ValueError("out must be [T, N]")
    opt = _lib.proj_options(False)
    st = lib.la_out_projection(_ptr(y), _ptr(weight), _ptr(out), T, K, N, _dtype(out.dtype),
                               ctypes.byref(opt), _stream(stream))
    _lib.check(st, "la_out_projection")
    _keep_for(stream, out)
    return out
