#!/usr/bin/env python3
"""Benchmark of the Lightning-Attention forward path on one MI355X.

One step = one gated bf16 prefill of the long-context workload
(B=1, T=1,048,576 tokens, 8 heads, head dim 128, RMSNorm*sigmoid gate):
feature map, blocking, chunk states and prefix, intra- and inter-block
products, state carry and the fused gate, i.e. every stage of the path, on
seeded synthetic inputs already resident in HBM.  The same run also times
the decode step (64 sequences x 64 heads x d=128, fp32 state, 1000 steps),
the CPU oracle on a bounded sample of the prefill workload, and the hybrid
model's softmax attention layer (32K tokens, a packed 512K-token batch and
1M tokens; 8 heads, rotary embedding on half of d = 128) with its own
matrix-core roofline and oracle baseline under "softmax_layer".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix-core peak, TFLOP/s
METRIC = "Lightning-attn prefill tokens/s + % bf16 MFMA peak; decode HBM GB/s"


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


class HipEvents:
    """Raw HIP events (libamdhip64) so the library can record them on its stream."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev.value
        self.n = n
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def close(self) -> None:
        """Destroy the events (before the runtime is torn down at exit)."""
        for i in range(self.n):
            if self.arr[i]:
                self.hip.hipEventDestroy(ctypes.c_void_p(self.arr[i]))
                self.arr[i] = None
        self.n = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def ptr(self, offset: int = 0) -> ctypes.c_void_p:
        return ctypes.c_void_p(ctypes.addressof(self.arr) + offset * ctypes.sizeof(ctypes.c_void_p))

    def record(self, i: int, stream: int) -> None:
        self.hip.hipEventRecord(ctypes.c_void_p(self.arr[i]), ctypes.c_void_p(stream))

    def elapsed_ms(self, a: int, b: int) -> float:
        self.hip.hipEventSynchronize(ctypes.c_void_p(self.arr[b]))
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.arr[a]),
                                        ctypes.c_void_p(self.arr[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def inputs_digest(torch, tensors, span=4 << 20):
    """sha256 of each input tensor's first and last `span` bytes (a fingerprint
    of the seeded inputs that costs no full copy to the host)."""
    import hashlib

    res = {}
    for name, t in tensors.items():
        if t is None:
            continue
        b = t.contiguous().view(torch.uint8).reshape(-1)
        h = hashlib.sha256()
        h.update(b[:span].cpu().numpy().tobytes())
        h.update(b[-span:].cpu().numpy().tobytes())
        res[name] = h.hexdigest()
    res["recipe"] = "sha256 of the first and last %d bytes of each tensor" % span
    return res


def bench_prefill(args, torch, lib, _lib, inputs, featurized=False, keep_rows=0):
    """The prefill step.  With ``featurized`` the same q, k, v values are
    passed as feature vectors already (the library's features-given mode: the
    feature map applied where they were produced), so the call skips SiLU.
    ``keep_rows``: a host copy of the output's first rows (of the last timed
    step) is returned for the parity leg."""
    w = inputs.WORKLOADS[args.workload]
    T, H, d = w.T, w.H, w.d
    log("generating %s inputs on the GPU (%s)" % (w.name, w.note))
    q, k, v, x = inputs.prefill_inputs(w, device="cuda")
    digest = inputs_digest(torch, {"q": q, "k": k, "v": v, "x": x})
    dev = q.device
    out = torch.empty((1, T, H * d), dtype=torch.float32, device=dev)
    state_out = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
    opt = _lib.options(block_size=args.block, gated=True, featurized=featurized)
    nbytes = lib.la_prefill_workspace_bytes(1, T, H, d, _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32,
                                            ctypes.byref(opt))
    ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
    plan = _lib.plan(False, 1, T, T, H, d, _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32, opt)
    chunk, names = plan.chunk_tokens, plan.kernel_names()
    nk = len(names)
    K, W = args.steps, args.warmup
    ev = HipEvents(2 * nk * (K + W))
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        opt.timing_events = ev.ptr(2 * nk * i)
        opt.n_timing = nk
        st = lib.la_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), x.data_ptr(), None, None,
                            None, out.data_ptr(), state_out.data_ptr(), None, 1, T, H, d,
                            _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32, ctypes.byref(opt),
                            ws.data_ptr(), ws.numel(), ctypes.c_void_p(stream))
        _lib.check(st, "la_prefill")

    tag = "prefill (features given)" if featurized else "prefill"
    log("%s: chunk %d tokens, kernels %s; %d warmup + %d timed steps" % (tag, chunk, names, W, K))
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    per_kernel = {}
    for j, name in enumerate(names):
        tot = 0.0
        for i in range(W, W + K):
            base = 2 * nk * i
            tot += ev.elapsed_ms(base + 2 * j, base + 2 * j + 1)
        per_kernel[name] = tot / K
    ev.close()
    log("%s: %.3f ms/step; kernels (ms): %s" %
        (tag, ms_step, ", ".join("%s %.3f" % kv for kv in per_kernel.items())))
    th = T * H
    res = {
        "T": T, "H": H, "d": d, "chunk": chunk, "block": plan.block_size,
        "fused_gate": bool(plan.fused_gate), "main_workgroups": plan.main_workgroups,
        "ms_per_step": ms_step,
        "tokens_per_s": T / (ms_step * 1e-3), "per_kernel_ms": per_kernel, "token_heads": th,
        "inputs_sha256": digest,
    }
    if keep_rows:
        res["out_head"] = out[0, :keep_rows].cpu()
    del q, k, v, x, out, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, lib, _lib, inputs):
    w = inputs.WORKLOADS["decode_64x64"]
    N, H, d, steps = w.N, w.H, w.d, args.decode_steps
    log("decode: generating state and %d steps of tokens on the GPU" % steps)
    S, z = inputs.decode_state(w, device="cuda")
    toks = [inputs.decode_token(w, s, device="cuda") for s in range(steps)]
    out = torch.empty((N, H * d), dtype=torch.float32, device="cuda")
    opt = _lib.options(block_size=64)
    ev = HipEvents(2 * steps + 2)
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    # default access (auto: streaming at this 256 MiB state), and the same
    # plain step with the state taken as cache-resident -- stepped back to back,
    # it stays in the 256 MB Infinity Cache, so that figure is not an HBM rate
    for key, normalized, access in (("plain", False, 0), ("normalized", True, 0),
                                    ("plain_cache_resident", False, 2)):
        opt.normalized = int(normalized)
        opt.state_access = access
        zz = z if normalized else None

        def call(s, timed):
            qs, ks, vs = toks[s]
            opt.timing_events = ev.ptr(2 * s) if timed else None
            opt.n_timing = 1 if timed else 0
            st = lib.la_decode_step(qs.data_ptr(), ks.data_ptr(), vs.data_ptr(), None, None,
                                    S.data_ptr(), None if zz is None else zz.data_ptr(),
                                    out.data_ptr(), N, H, d, _lib.LA_DTYPE_BF16,
                                    _lib.LA_DTYPE_F32, ctypes.byref(opt), None, 0,
                                    ctypes.c_void_p(stream))
            _lib.check(st, "la_decode_step")

        for s in range(min(10, steps)):
            call(s, False)
        torch.cuda.synchronize()
        # three trials of `steps` back-to-back steps: per-step kernel times
        # (HIP events around each launch), loop time and host wall time
        per_step, loops, walls = [], [], []
        for _trial in range(3):
            ev.record(2 * steps, stream)
            t0 = time.perf_counter()
            for s in range(steps):
                call(s, True)
            ev.record(2 * steps + 1, stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            per_step += [ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(steps)]
            loops.append(ev.elapsed_ms(2 * steps, 2 * steps + 1) / steps)
            walls.append((t1 - t0) / steps)
        per_step.sort()
        kern = per_step[len(per_step) // 2]
        kern_mean = sum(per_step) / len(per_step)
        loop = sorted(loops)[1]
        wall = sorted(walls)[1]
        # algorithmic bytes per step: S read + write, z read + write, q/k/v in, y out
        nbytes = 2 * N * H * d * d * 4 + 3 * N * H * d * 2 + N * H * d * 4
        if normalized:
            nbytes += 2 * N * H * d * 4
        res[key] = {
            "kernel_us": kern * 1e3, "kernel_us_mean": kern_mean * 1e3,
            "loop_us_per_step": loop * 1e3, "trials": 3, "steps_per_trial": steps,
            "wall_us_per_step": wall * 1e6, "bytes_per_step": nbytes,
            "GBps": nbytes / (kern * 1e-3) / 1e9, "hbm_frac": nbytes / (kern * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "state_access": ["auto (streaming: non-temporal, contiguous per sequence-head)", "streaming",
                             "cache-resident (not an HBM rate: the state stays in the Infinity Cache)"][access],
        }
        log("decode %s: kernel %.1f us/step median of %d (%.0f GB/s), loop %.1f us/step" %
            (key, kern * 1e3, len(per_step), res[key]["GBps"], loop * 1e3))
    ev.close()
    del toks, S, z
    torch.cuda.empty_cache()
    res["cold"] = bench_decode_cold(args, torch, lib, _lib, inputs)
    return res


def bench_decode_cold(args, torch, lib, _lib, inputs, pools=4):
    """The decode step with its state out of the Infinity Cache: step s
    works on state pool s % pools (each the workload's 64 x 64 x 128 x 128
    fp32 state, 256 MiB), so between two visits to a pool the other pools
    stream 768 MiB through the 256 MB cache.  Plain mode, per-step kernel
    times from HIP events."""
    w = inputs.WORKLOADS["decode_64x64"]
    N, H, d, steps = w.N, w.H, w.d, args.decode_steps
    S0, _ = inputs.decode_state(w, device="cuda")
    Ss = [S0.clone() for _ in range(pools)]
    del S0
    toks = [inputs.decode_token(w, s, device="cuda") for s in range(min(steps, 64))]
    out = torch.empty((N, H * d), dtype=torch.float32, device="cuda")
    opt = _lib.options(block_size=64)
    stream = torch.cuda.current_stream().cuda_stream
    per_step = []
    with HipEvents(2 * steps) as ev:
        def call(s, timed):
            qs, ks, vs = toks[s % len(toks)]
            opt.timing_events = ev.ptr(2 * s) if timed else None
            opt.n_timing = 1 if timed else 0
            st = lib.la_decode_step(qs.data_ptr(), ks.data_ptr(), vs.data_ptr(), None, None,
                                    Ss[s % pools].data_ptr(), None, out.data_ptr(), N, H, d,
                                    _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32, ctypes.byref(opt),
                                    None, 0, ctypes.c_void_p(stream))
            _lib.check(st, "la_decode_step")

        for s in range(2 * pools):
            call(s, False)
        torch.cuda.synchronize()
        for _trial in range(3):
            for s in range(steps):
                call(s, True)
            torch.cuda.synchronize()
            per_step += [ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(steps)]
    per_step.sort()
    kern = per_step[len(per_step) // 2]
    nbytes = 2 * N * H * d * d * 4 + 3 * N * H * d * 2 + N * H * d * 4
    gbs = nbytes / (kern * 1e-3) / 1e9
    log("decode cold (%d rotating state pools, %d MiB): kernel %.1f us/step (%.0f GB/s)"
        % (pools, pools * N * H * d * d * 4 >> 20, kern * 1e3, gbs))
    del Ss, toks, out
    torch.cuda.empty_cache()
    return {"pools": pools, "state_bytes_total": pools * N * H * d * d * 4,
            "kernel_us": kern * 1e3, "steps": 3 * steps, "bytes_per_step": nbytes, "GBps": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS,
            "note": "step s updates state pool s %% %d in place: each pool is the decode "
                    "workload's 256 MiB state, so consecutive visits to a pool are 768 MiB of "
                    "other state traffic apart and the 256 MB Infinity Cache cannot hold it"
                    % pools}


def bench_other_prefill(args, torch, api, inputs):
    """The 32K-token, packed-varlen and 4M-token workloads through the Python binding:
    whole-call time (HIP events on the current stream), median over repeats."""
    res = {}
    for name, reps in (("prefill_32k", 100), ("varlen_512k", 20), ("prefill_4m", 5)):
        w = inputs.WORKLOADS[name]
        if w.kind == "prefill":
            q, k, v, x = inputs.prefill_inputs(w, device="cuda")
            run = lambda: api.la_prefill(q, k, v, x)
            tokens = w.T
        else:
            q, k, v, x, cu = inputs.varlen_inputs(w, device="cuda")
            cu_d = cu.cuda()
            maxlen = int((cu[1:] - cu[:-1]).max())
            run = lambda: api.la_prefill_varlen(q, k, v, cu_d, maxlen, x)
            tokens = w.total_T
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
        times.sort()
        med = times[len(times) // 2]
        th = tokens * w.H
        res[name] = {"ms_median": med, "ms_p10": times[len(times) // 10],
                     "ms_p90": times[(9 * len(times)) // 10], "tokens_per_s": tokens / (med * 1e-3),
                     "path_min_bytes_GBps": th * 1536 / (med * 1e-3) / 1e9,
                     "note": "whole call incl. workspace allocation in the binding; " + w.note}
        log("%s: %.3f ms median (p10 %.3f, p90 %.3f), %.0f tokens/s" %
            (name, med, res[name]["ms_p10"], res[name]["ms_p90"], res[name]["tokens_per_s"]))
        del q, k, v, x
        torch.cuda.empty_cache()
    return res


def bench_serving(args, torch, api, inputs, reps=50):
    """One serving step (64 decode tokens + a 32704-token prompt chunk, all
    continuing from pool rows) run four ways, median over repeats (HIP events):
      two_streams   la_serve_step, decode tokens and the chunk on two streams;
      serve_one_stream   la_serve_step with both parts on one stream (decode
                    first; decode_ms is then the whole step);
      one_stream    the decode call, then the prefill call, on one stream;
      one_call      every row as one packed varlen call (the decode tokens as
                    length-1 sequences);
      decode_alone / chunk_alone   each part by itself.
    decode_ms is the time from the step's start until the decode tokens'
    outputs are written; step_ms until the whole step is done.  The pool is
    updated in place each repeat (timing only).  Two views: "wall" starts the
    clock when the host begins submitting the step (host submission in the
    binding included); "device" first holds the stream with a spin kernel
    until the host has submitted the whole step, so only device time counts."""
    w = inputs.WORKLOADS["serve_mixed_32k"]
    q, k, v, x, pool = inputs.serve_inputs(w, device="cuda")
    nd, rows = w.N, w.total_T
    dev = q.device
    dslots = torch.arange(nd, dtype=torch.int32, device=dev)
    pslots = torch.tensor([nd], dtype=torch.int32, device=dev)
    pcu = torch.tensor([0, rows - nd], dtype=torch.int32, device=dev)
    all_slots = torch.arange(nd + 1, dtype=torch.int32, device=dev)
    all_cu = torch.tensor(list(range(nd + 1)) + [rows], dtype=torch.int32, device=dev)
    cur = torch.cuda.current_stream()
    s_dec, s_pre = torch.cuda.Stream(), torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # spin-kernel cycles for ~2 ms of hold, from one timed spin
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(cur)
    torch.cuda._sleep(1 << 20)
    b.record(cur)
    b.synchronize()
    hold_cycles = int((1 << 20) * 2.0 / max(a.elapsed_time(b), 1e-3))
    hold = [False]
    log("serving: device view holds the stream %d spin cycles (~2 ms)" % hold_cycles)

    def start():
        if hold[0]:
            torch.cuda._sleep(hold_cycles)
        a = ev()
        a.record(cur)
        return a

    def two_streams():
        a, e_dec, e_pre = start(), ev(), ev()
        s_dec.wait_stream(cur)
        s_pre.wait_stream(cur)
        api.la_serve_step(q, k, v, pool, dslots, pcu, pslots, rows - nd, x=x,
                          decode_stream=s_dec, prefill_stream=s_pre)
        e_dec.record(s_dec)
        e_pre.record(s_pre)
        cur.wait_stream(s_dec)
        cur.wait_stream(s_pre)
        return a, e_dec, (e_dec, e_pre)

    def serve_one_stream():
        a, e_end = start(), ev()
        api.la_serve_step(q, k, v, pool, dslots, pcu, pslots, rows - nd, x=x,
                          decode_stream=cur, prefill_stream=cur)
        e_end.record(cur)
        return a, e_end, (e_end,)

    def one_stream():
        a, e_dec, e_end = start(), ev(), ev()
        api.la_decode_step(q[:nd], k[:nd], v[:nd], pool, x=x[:nd], state_slots=dslots)
        e_dec.record(cur)
        api.la_prefill_varlen(q[nd:], k[nd:], v[nd:], pcu, rows - nd, x[nd:], None, pool,
                              state_slots=pslots)
        e_end.record(cur)
        return a, e_dec, (e_end,)

    def one_call():
        a, e_end = start(), ev()
        api.la_prefill_varlen(q, k, v, all_cu, rows - nd, x, None, pool, state_slots=all_slots)
        e_end.record(cur)
        return a, e_end, (e_end,)

    def decode_alone():
        a, e_end = start(), ev()
        api.la_decode_step(q[:nd], k[:nd], v[:nd], pool, x=x[:nd], state_slots=dslots)
        e_end.record(cur)
        return a, e_end, (e_end,)

    def chunk_alone():
        a, e_end = start(), ev()
        api.la_prefill_varlen(q[nd:], k[nd:], v[nd:], pcu, rows - nd, x[nd:], None, pool,
                              state_slots=pslots)
        e_end.record(cur)
        return a, e_end, (e_end,)

    res = {"workload": w.note, "reps": reps}
    from linear_attention_long_amd import _lib
    opt = _lib.options(0, False, True, 0, 1e-6, 0)
    for name, nseq, maxlen in (("one_call", nd + 1, rows - nd), ("chunk_alone", 1, rows - nd)):
        p = _lib.plan(True, nseq, rows if nseq > 1 else rows - nd, maxlen, w.H, w.d,
                      _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32, opt)
        res["plan_" + name] = {"fused_gate": bool(p.fused_gate), "chunk_tokens": p.chunk_tokens,
                               "main_workgroups": p.main_workgroups,
                               "kernels": p.kernel_names()}
        log("serving %s plan: %s" % (name, res["plan_" + name]))
    for view in ("wall", "device"):
        hold[0] = view == "device"
        res[view] = {}
        for name, fn in (("two_streams", two_streams), ("serve_one_stream", serve_one_stream),
                         ("one_stream", one_stream),
                         ("one_call", one_call), ("decode_alone", decode_alone),
                         ("chunk_alone", chunk_alone)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            dts, sts = [], []
            for _ in range(reps):
                a, e_dec, ends = fn()
                torch.cuda.synchronize()
                dts.append(a.elapsed_time(e_dec))
                sts.append(max(a.elapsed_time(e) for e in ends))
            dts.sort()
            sts.sort()
            res[view][name] = {"decode_ms": dts[reps // 2], "step_ms": sts[reps // 2],
                               "step_ms_p90": sts[(9 * reps) // 10]}
            log("serving (%s) %s: decode tokens ready %.4f ms, step %.4f ms (median)"
                % (view, name, dts[reps // 2], sts[reps // 2]))
    del q, k, v, x, pool
    torch.cuda.empty_cache()
    return res


# (workload, timed calls, precision): 1 = split operands in both products
# (the library's default, within 1e-2 of the output's rms for any bf16
# input), 2 = fp16 operands (q, k, v, probabilities), 0 = single bf16 operands
SOFTMAX_WORKLOADS = (("softmax_32k", 10, 1), ("softmax_varlen_512k", 3, 1), ("softmax_1m", 1, 1),
                     ("softmax_32k", 10, 2), ("softmax_varlen_512k", 3, 2),
                     ("softmax_32k", 20, 0), ("softmax_varlen_512k", 5, 0))
SOFTMAX_KEY = {1: "", 2: "_fp16", 0: "_single"}
SOFTMAX_NOTE = {
    1: ("split bf16 hi+lo operands in both products (default; within 1e-2 of the output's rms "
        "for any bf16 input)"),
    2: ("fp16 operands (q, k, v times 2^-6 and the probabilities rounded to fp16, one product "
        "each): about 3e-3 to 5e-3 of the output's rms for scores of unit spread and more, "
        "growing with the spread (not the library default)"),
    0: ("single bf16 operands: about 1e-3 of the values' scale, which on long rows exceeds "
        "the 1e-2-of-output-rms bound for bf16 inputs (not the library default)"),
}


def softmax_flops(cu):
    """Algorithmic flops of causal attention per head-independent unit: QK^T and
    P V over the d features for every (query, key <= query) pair of each
    sequence, 4 d flops per pair and head."""
    L = (cu[1:] - cu[:-1]).to(dtype=__import__("torch").int64)
    return int((L * (L + 1) // 2).sum())


def bench_softmax(args, torch, lib, _lib, inputs):
    """The hybrid model's softmax attention layer (include/la_softmax.h) on its
    workloads: per-kernel times from HIP events on the call's stream."""
    res = {}
    for name, reps, prec in SOFTMAX_WORKLOADS:
        if name == "softmax_1m" and args.no_softmax_1m:
            continue
        key = name + SOFTMAX_KEY[prec]
        w = inputs.WORKLOADS[name]
        q, k, v, cu = inputs.softmax_inputs(w, device="cuda")
        cud = cu.cuda()
        T, H, d = q.shape
        Hkv = k.shape[1]
        nseq = cu.numel() - 1
        maxlen = int((cu[1:] - cu[:-1]).max())
        pairs = softmax_flops(cu)
        flops = 4.0 * d * H * pairs
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
        opt = _lib.softmax_options(w.extra["rotary_dim"], w.extra["rope_base"], 0.0, prec)
        nbytes = lib.la_softmax_workspace_bytes(nseq, T, maxlen, H, Hkv, d, _lib.LA_DTYPE_BF16,
                                                _lib.LA_DTYPE_BF16, ctypes.byref(opt))
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")
        names = (["plan"] if nseq > 1 else []) + ["rotate", "attention"]
        nk = len(names)
        ev = HipEvents(2 * nk * (reps + 1))
        stream = torch.cuda.current_stream().cuda_stream

        def call(i):
            opt.timing_events = ev.ptr(2 * nk * i)
            opt.n_timing = nk
            st = lib.la_softmax_attention_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 cud.data_ptr(), nseq, T, maxlen, H, Hkv, d,
                                                 _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_BF16,
                                                 out.data_ptr(), None, ctypes.byref(opt),
                                                 ws.data_ptr(), ws.numel(), ctypes.c_void_p(stream))
            _lib.check(st, "la_softmax_attention_varlen")

        call(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(1, reps + 1):
            call(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / reps
        per = {}
        for j, kn in enumerate(names):
            per[kn] = sum(ev.elapsed_ms(2 * nk * i + 2 * j, 2 * nk * i + 2 * j + 1)
                          for i in range(1, reps + 1)) / reps
        ev.close()
        att = per["attention"]
        res[key] = {"tokens": T, "sequences": nseq, "max_seqlen": maxlen, "H": H, "Hkv": Hkv,
                    "d": d, "rotary_dim": w.extra["rotary_dim"], "rope_base": w.extra["rope_base"],
                    "precision": SOFTMAX_NOTE[prec],
                    "ms_per_call": ms, "per_kernel_ms": per, "algorithmic_flops": flops,
                    "attention_TFLOPs": flops / (att * 1e-3) / 1e12,
                    "call_TFLOPs": flops / (ms * 1e-3) / 1e12,
                    "tokens_per_s": T / (ms * 1e-3), "reps": reps}
        log("softmax %s: %.3f ms/call (attention kernel %.3f ms, %.0f TFLOP/s = %.1f%% of "
            "the bf16 peak)" % (key, ms, att, res[key]["attention_TFLOPs"],
                                100 * res[key]["attention_TFLOPs"] / MFMA_BF16_PEAK_TFS))
        del q, k, v, cud, out, ws
        torch.cuda.empty_cache()
    return res


def bench_projection(args, torch, lib, _lib, inputs):
    """The layer's projections (include/la_proj.h): the input GEMM kernel on
    proj_32k (HIP events around each launch; algorithmic flops 2 T K 4F) and
    the output GEMM on the same layer's output side (2 T F K); the layer's
    input side end to end on 32K and 1M tokens (the projection with SiLU in
    its epilogue followed by the path in its features-given mode, against the
    raw projection followed by the path's own SiLU), and the whole layer with
    the output projection after the path."""
    from linear_attention_long_amd import api

    res = {}
    w = inputs.WORKLOADS["proj_32k"]
    h, wt = inputs.projection_inputs(w, device="cuda")
    T, K = h.shape
    H, d = w.H, w.d
    F = H * d
    outs = [torch.empty((T, F), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    reps = 20
    stream = torch.cuda.current_stream().cuda_stream
    opt = _lib.proj_options(True)
    with HipEvents(2 * (reps + 1)) as ev:
        def call(i):
            opt.timing_events = ev.ptr(2 * i)
            opt.n_timing = 1
            st = lib.la_qkvx_projection(h.data_ptr(), wt.data_ptr(), outs[0].data_ptr(),
                                        outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(),
                                        T, K, F, _lib.LA_DTYPE_BF16, ctypes.byref(opt),
                                        ctypes.c_void_p(stream))
            _lib.check(st, "la_qkvx_projection")

        call(0)
        torch.cuda.synchronize()
        for i in range(1, reps + 1):
            call(i)
        torch.cuda.synchronize()
        times = sorted(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(1, reps + 1))
    ms = times[len(times) // 2]
    flops = 2.0 * T * K * 4 * F
    tfs = flops / (ms * 1e-3) / 1e12
    res["kernel"] = {"workload": w.name, "T": T, "K": K, "F": F, "out": "bf16 q, k, v (SiLU), gate",
                     "kernel_ms": ms, "kernel_ms_mean": sum(times) / len(times),
                     "algorithmic_flops": flops, "TFLOPs": tfs,
                     "mfma_bf16_peak_frac": tfs / MFMA_BF16_PEAK_TFS, "reps": reps}
    log("projection %s: %.3f ms, %.0f TFLOP/s = %.1f%% of the bf16 peak"
        % (w.name, ms, tfs, 100 * tfs / MFMA_BF16_PEAK_TFS))
    del outs

    # the output projection: y [T, F] bf16 times W_o [K, F]^T -> [T, K] bf16
    yo, wo = inputs.out_projection_inputs(w, device="cuda")
    zo = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    oopt = _lib.proj_options(False)
    with HipEvents(2 * (reps + 1)) as ev:
        def ocall(i):
            oopt.timing_events = ev.ptr(2 * i)
            oopt.n_timing = 1
            st = lib.la_out_projection(yo.data_ptr(), wo.data_ptr(), zo.data_ptr(), T, F, K,
                                       _lib.LA_DTYPE_BF16, ctypes.byref(oopt),
                                       ctypes.c_void_p(stream))
            _lib.check(st, "la_out_projection")

        ocall(0)
        torch.cuda.synchronize()
        for i in range(1, reps + 1):
            ocall(i)
        torch.cuda.synchronize()
        otimes = sorted(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(1, reps + 1))
    oms = otimes[len(otimes) // 2]
    oflops = 2.0 * T * F * K
    otfs = oflops / (oms * 1e-3) / 1e12
    res["out_kernel"] = {"workload": w.name + " output side", "T": T, "K_in": F, "N": K,
                         "out": "bf16 partial sum of the layer output (this device's heads)",
                         "kernel_ms": oms, "kernel_ms_mean": sum(otimes) / len(otimes),
                         "algorithmic_flops": oflops, "TFLOPs": otfs,
                         "mfma_bf16_peak_frac": otfs / MFMA_BF16_PEAK_TFS, "reps": reps}
    log("output projection %s: %.3f ms, %.0f TFLOP/s = %.1f%% of the bf16 peak"
        % (w.name, oms, otfs, 100 * otfs / MFMA_BF16_PEAK_TFS))
    del yo, zo

    layer = {}
    for name, nrep in (("proj_32k", 10), ("proj_1m", 3)):
        wl = inputs.WORKLOADS[name]
        if name != w.name:
            del h, wt
            torch.cuda.empty_cache()
            h, wt = inputs.projection_inputs(wl, device="cuda")
        T = h.shape[0]
        o4 = [torch.empty((T, F), dtype=torch.bfloat16, device="cuda") for _ in range(4)]

        def side(feat):
            q, k, v, xg = api.la_qkvx_projection(h, wt, F, featurize=feat, out=o4)
            return api.la_prefill(q.view(1, T, H, d), k.view(1, T, H, d), v.view(1, T, H, d),
                                  xg.view(1, T, F), featurized=feat, return_state=False)[0]

        z = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")

        def whole():
            q, k, v, xg = api.la_qkvx_projection(h, wt, F, featurize=True, out=o4)
            y = api.la_prefill(q.view(1, T, H, d), k.view(1, T, H, d), v.view(1, T, H, d),
                               xg.view(1, T, F), featurized=True, out_dtype=torch.bfloat16,
                               return_state=False)[0]
            return api.la_out_projection(y.view(T, F), wo, out=z)

        entry = {}
        for key, fn in (("silu_in_projection", lambda: side(True)),
                        ("silu_in_path", lambda: side(False)), ("whole_layer", whole)):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(nrep):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                b.synchronize()
                ts.append(a.elapsed_time(b))
            ts.sort()
            entry[key + "_ms"] = ts[len(ts) // 2]
        entry["tokens"] = T
        entry["tokens_per_s_silu_in_projection"] = T / (entry["silu_in_projection_ms"] * 1e-3)
        entry["tokens_per_s_whole_layer"] = T / (entry["whole_layer_ms"] * 1e-3)
        entry["whole_layer_note"] = ("input projection (SiLU in the epilogue), the path (features "
                                     "given, gated, bf16 out), output projection; whole calls "
                                     "through the binding")
        layer[name] = entry
        log("layer input side %s: projection + path %.3f ms with SiLU in the projection's "
            "epilogue, %.3f ms with SiLU in the path; whole layer with the output projection "
            "%.3f ms" % (name, entry["silu_in_projection_ms"], entry["silu_in_path_ms"],
                         entry["whole_layer_ms"]))
        del o4, z
        torch.cuda.empty_cache()
    res["layer_input_side"] = layer
    del h, wt, wo
    torch.cuda.empty_cache()
    return res


def cpu_baseline_softmax(inputs, rows=256):
    """The softmax-layer oracle (plain fp64 C) on the last `rows` tokens of the
    32K-token workload, every head: algorithmic TFLOP/s."""
    import numpy as np

    from oracle import softmax as SO

    w = inputs.WORKLOADS["softmax_32k"]
    q, k, v, cu = (t.cpu() for t in inputs.softmax_inputs(w, device="cuda"))  # the bench's values
    T, H, d = q.shape
    toks = np.repeat(np.arange(T - rows, T), H)
    heads = np.tile(np.arange(H), rows)
    threads = min(os.cpu_count() or 1, 16)
    t0 = time.perf_counter()
    SO.attention(q, k, v, cu, rotary_dim=w.extra["rotary_dim"], rope_base=w.extra["rope_base"],
                 rows=toks, heads=heads, nthreads=threads)
    dt = time.perf_counter() - t0
    flops = 4.0 * d * float((toks + 1).sum())
    log("cpu baseline (softmax layer): %.2f s for %d token-heads" % (dt, len(toks)))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "last %d tokens x %d heads of softmax_32k (each over its %d-%d keys); fp64 "
                      "per-pair loops; %.1f s" % (rows, H, T - rows + 1, T, dt)}


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy rate (read + write bytes per second) on this GPU."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    b.synchronize()
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def calibrate_copy(args, torch):
    """A plain copy of a known number of bytes: under a byte counter, its
    reading per dispatch against the bytes it must move gives the counter's
    scale."""
    n = args.calibrate_copy
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    log("copy of %d bytes: %.3f ms, %.0f GB/s read+write" % (n, dt * 1e3, 2 * n / dt / 1e9))
    print(json.dumps({"copy_bytes": n, "steps": args.steps, "ms": dt * 1e3}), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "main_gated_prefill_1m_traffic.md")
SOFTMAX_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "softmax_attention_32k_traffic.md")
PROJECTION_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "projection_gemm_32k_traffic.md")
SOURCES = os.path.join(ROOT, "linear_attention_long_amd", "csrc")


def code_text(src: str) -> str:
    """C/C++ source without its comments and blank lines: each comment
    becomes one space (a line comment ends at its newline), string and
    character literals are kept as written, trailing blanks are cut and
    empty lines dropped.  Edits to comments or blank lines leave it as it
    is; any change to the code changes it."""
    out = []
    i, n = 0, len(src)
    while i < n:
        ch = src[i]
        if ch in "\"'":
            j = i + 1
            while j < n and src[j] != ch and src[j] != "\n":
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def _digest(names) -> str:
    """sha256 over the names and code (code_text: comments and blank lines
    left out) of the given csrc/ files, in order."""
    import hashlib

    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        h.update(code_text(open(os.path.join(SOURCES, name), encoding="utf-8").read()).encode())
    return h.hexdigest()


def source_digest() -> str:
    """sha256 over the linear-attention kernels' HIP sources (names and
    contents of csrc/la_*, sorted)."""
    return _digest(sorted(n for n in os.listdir(SOURCES)
                          if n.startswith("la_") and n.endswith((".h", ".hip"))))


def softmax_source_digest() -> str:
    """sha256 over the sources the softmax kernels are built from."""
    return _digest(("la_device.h", "sm_api.hip", "sm_kernels.h"))


def projection_source_digest() -> str:
    """sha256 over the sources the projection GEMM is built from."""
    return _digest(("la_device.h", "proj_api.hip", "proj_kernels.h"))


def committed_traffic(path, digest, key="hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed counter summary (its `key`
    line), or None when the file is missing or its `source_sha256` line no
    longer matches `digest` (the kernel changed since the counters were
    taken)."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith(("source_sha256", key)):
            k, val = line.strip().strip("`").split(":", 1)
            vals[k.strip()] = val.strip().strip("`")
    if vals.get("source_sha256") != digest or key not in vals:
        return None
    return float(vals[key])


def measured_traffic():
    """HBM bytes per launch of the fused main pass (1M-token prefill)."""
    return committed_traffic(TRAFFIC_FILE, source_digest())


def measured_softmax_traffic():
    """HBM bytes per launch of the softmax attention kernel (32K, default mode)."""
    return committed_traffic(SOFTMAX_TRAFFIC_FILE, softmax_source_digest())


def measured_projection_traffic(side="in"):
    """HBM bytes per launch of the projection GEMM at proj_32k, input side
    ("in") or output side ("out")."""
    key = "hbm_bytes_per_launch" if side == "in" else "hbm_bytes_per_launch_out"
    return committed_traffic(PROJECTION_TRAFFIC_FILE, projection_source_digest(), key)


def cpu_baseline(args, inputs, gpu_head=None):
    """The oracle (plain fp64 C) on the first tokens of the same workload.
    With ``gpu_head`` (the benched call's output for those tokens, on the
    host) it also reports the parity of the benched configuration: causal,
    so the first tokens' outputs do not depend on the rest."""
    import numpy as np
    import torch

    from oracle import oracle as O

    w = inputs.WORKLOADS[args.workload]
    T = args.cpu_tokens
    # the benched call's own inputs, cut to their first T tokens (a shorter
    # draw on the GPU would not be a prefix of them)
    q, k, v, x = inputs.prefill_inputs(w, device="cuda")
    q, k, v, x = (t[:, :T].cpu() for t in (q, k, v, x))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    threads = min(os.cpu_count() or 1, w.H)
    log("cpu baseline: oracle on %d tokens x %d heads with %d threads" % (T, w.H, threads))
    t0 = time.perf_counter()
    ref, _, _ = O.forward(q[0], k[0], v[0], x[0], gated=True, nthreads=threads)
    dt = time.perf_counter() - t0
    log("cpu baseline: %.2f s -> %.0f tokens/s" % (dt, T / dt))
    res = {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "first %d tokens of the %s workload, all %d heads, gated; fp64 "
                     "token-by-token recurrence; %.1f s" % (T, w.name, w.H, dt)}
    parity = None
    if gpu_head is not None:
        got = gpu_head.numpy().astype(np.float64)
        err = float(np.abs(got - ref).max() / np.sqrt(np.mean(ref * ref)))
        parity = {"max_abs_err_over_rms": err, "bound": 1e-2, "pass": bool(err <= 1e-2),
                  "elements": int(ref.size),
                  "compared": "every output of the first %d tokens (all %d heads) of the benched "
                              "call against the oracle above" % (T, w.H)}
        log("parity of the benched call: max|err|/rms %.2e over %d outputs" % (err, ref.size))
    return res, parity


def features_given_summary(feat, main_name):
    """The same workload with q, k, v passed as features (SiLU applied where
    they were produced, e.g. in the projection's epilogue): per-kernel times
    and the main pass's HBM fraction on the same algorithmic bytes."""
    th = feat["token_heads"]
    unit = 4 * 256 + 512 if main_name == "main_gated" else 3 * 256 + 512
    nbytes = th * unit
    if feat["T"] > feat["chunk"]:
        nbytes += feat["main_workgroups"] * feat["d"] * feat["d"] * 4
    ms = feat["per_kernel_ms"].get(main_name)
    gbs = None if not ms else nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_step": feat["ms_per_step"], "tokens_per_s": feat["tokens_per_s"],
            "per_kernel_ms": feat["per_kernel_ms"], "main_GBps": gbs,
            "main_hbm_frac": None if gbs is None else gbs / HBM_PEAK_GBS,
            "note": "same inputs taken as feature vectors: no SiLU in the path, exact single "
                    "bf16 products for phi(q).phi(k), P.V's value side, Q.S's query side and "
                    "the state update"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_1m", choices=["prefill_1m", "prefill_32k"])
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-featurized", action="store_true",
                    help="skip the prefill with inputs given as features")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 32K-token and varlen timings and the copy-bandwidth reference")
    ap.add_argument("--cpu-tokens", type=int, default=524288)
    ap.add_argument("--no-softmax", action="store_true",
                    help="skip the softmax attention layer's workloads")
    ap.add_argument("--no-softmax-1m", action="store_true",
                    help="skip its 1M-token workload (about 2 s per call)")
    ap.add_argument("--softmax-only", action="store_true",
                    help="only time the softmax layer's workloads (for profiling its kernels); "
                         "prints their JSON instead of the benchmark line")
    ap.add_argument("--no-projection", action="store_true",
                    help="skip the input projection GEMM and the layer input side")
    ap.add_argument("--projection-only", action="store_true",
                    help="only time the input projection (prints its JSON)")
    ap.add_argument("--block", type=int, default=0, help="block size (0 = library default)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes --steps times "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU code (the path "
              "shards by head or by sequence with no collective).  Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from linear_attention_long_amd import _lib, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args, torch)
        return
    lib = _lib.load()
    log("device: %s" % torch.cuda.get_device_name(0))
    if args.projection_only:
        print(json.dumps({"projection": bench_projection(args, torch, lib, _lib, inputs)}),
              flush=True)
        return
    if args.softmax_only:
        print(json.dumps({"softmax_layer": bench_softmax(args, torch, lib, _lib, inputs)}),
              flush=True)
        return

    keep = 0 if args.no_cpu_baseline else args.cpu_tokens
    pre = bench_prefill(args, torch, lib, _lib, inputs, keep_rows=keep)
    head = pre.pop("out_head", None)
    feat = None if args.no_featurized else bench_prefill(args, torch, lib, _lib, inputs,
                                                         featurized=True)
    dec = None if args.no_decode else bench_decode(args, torch, lib, _lib, inputs)
    other = serve = None
    if not args.no_extra:
        from linear_attention_long_amd import api

        other = bench_other_prefill(args, torch, api, inputs)
        serve = bench_serving(args, torch, api, inputs)
        if dec is not None:
            cgbs = copy_bandwidth(torch)
            log("device copy: %.0f GB/s" % cgbs)
            for key in dec:
                dec[key]["device_copy_GBps"] = cgbs
                dec[key]["frac_of_copy"] = dec[key]["GBps"] / cgbs
    proj = None if args.no_projection else bench_projection(args, torch, lib, _lib, inputs)
    cpu, parity = (None, None) if args.no_cpu_baseline else cpu_baseline(args, inputs, head)
    del head
    soft = None
    if not args.no_softmax:
        soft = bench_softmax(args, torch, lib, _lib, inputs)
        lead = soft["softmax_32k"]   # the default (split-operand) mode
        att_ms = lead["per_kernel_ms"]["attention"]
        soft_traffic = measured_softmax_traffic()
        soft = {
            "workloads": soft,
            "roofline": {"bound": "mfma",
                         "kernel": "attention (k_sm_attn), softmax_32k, split operands (default)",
                         "achieved": lead["attention_TFLOPs"], "peak": MFMA_BF16_PEAK_TFS,
                         "unit": "TFLOP/s", "frac": lead["attention_TFLOPs"] / MFMA_BF16_PEAK_TFS,
                         "traffic": soft_traffic,
                         "algorithmic_flops_per_launch": lead["algorithmic_flops"],
                         "avg_launch_ms": att_ms},
            "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_softmax(inputs),
        }
        if "softmax_1m" in soft["workloads"] and args.workload == "prefill_1m":
            soft["softmax_over_linear_1m"] = (soft["workloads"]["softmax_1m"]["ms_per_call"]
                                              / pre["ms_per_step"])

    th = pre["token_heads"]
    if pre["fused_gate"]:
        # main pass with the gate fused: reads q, k, v, x (4 x 256 B bf16) and
        # writes the fp32 output (512 B) per token-head
        main_name, main_kernel, main_unit = "main_gated", "main pass + gate (k_prefill_fused)", 4 * 256 + 512
    else:
        # main pass alone: reads q, k, v (3 x 256 B bf16), writes fp32 Y (512 B)
        main_name, main_kernel, main_unit = "main", "main pass (k_prefill_main)", 3 * 256 + 512
    main_ms = pre["per_kernel_ms"][main_name]
    main_bytes = th * main_unit
    if pre["T"] > pre["chunk"]:
        # plus the fp32 d x d state each (chunk, head) workgroup starts from
        main_bytes += pre["main_workgroups"] * pre["d"] * pre["d"] * 4
    main_gbs = main_bytes / (main_ms * 1e-3) / 1e9
    # whole path, minimal traffic: q, k, v, x in (bf16) and fp32 out = 1536 B per token-head
    path_bytes = th * 1536
    path_gbs = path_bytes / (pre["ms_per_step"] * 1e-3) / 1e9
    # algorithmic flops per token-head at block B, head dim d: intra 2(B+1)d
    # (causal half of the block for phi(Q)phi(K)^T and P.V), inter 2d^2, state 2d^2
    B, d = pre["block"], pre["d"]
    flops = th * (2 * (B + 1) * d + 4 * d * d)
    tflops = flops / (pre["ms_per_step"] * 1e-3) / 1e12
    # the same count at the pages' block of 256 tokens (131,328 per token-head
    # at d = 128): more intra-block work for the same result
    tflops256 = th * (2 * 257 * d + 4 * d * d) / (pre["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: bf16 q/k/v N(0,1)/sqrt(128), B=1 T=%d H=%d d=%d, block %d, "
                               "fp32 state carry, RMSNorm*sigmoid gate, fp32 out"
                               % (args.workload, pre["T"], pre["H"], pre["d"], pre["block"]),
                   "global_batch": 1, "seq_len": pre["T"], "heads": pre["H"], "head_dim": pre["d"],
                   "block": pre["block"], "chunk_tokens": pre["chunk"],
                   "fused_gate": pre["fused_gate"]},
        "roofline": {"bound": "hbm", "kernel": main_kernel,
                     "achieved": main_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": main_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if main_name == "main_gated" else None,
                     "algorithmic_bytes_per_launch": main_bytes,
                     "avg_launch_ms": main_ms},
        "cpu_baseline": cpu,
        "parity": parity,
        "prefill": {"per_kernel_ms": pre["per_kernel_ms"], "path_min_bytes_GBps": path_gbs,
                    "inputs_sha256": pre["inputs_sha256"],
                    "path_hbm_roofline_frac": path_gbs / HBM_PEAK_GBS,
                    "algorithmic_TFLOPs": tflops, "mfma_bf16_peak_frac": tflops / MFMA_BF16_PEAK_TFS,
                    "flops_per_token_head": 2 * (B + 1) * d + 4 * d * d,
                    "algorithmic_TFLOPs_at_block_256": tflops256,
                    "mfma_bf16_peak_frac_at_block_256": tflops256 / MFMA_BF16_PEAK_TFS},
        "decode": dec,
        "other_prefill": other,
        "serving_step": serve,
        "softmax_layer": soft,
        "projection": None if proj is None else {
            "roofline": {"bound": "mfma", "kernel": "input projection GEMM (k_proj), proj_32k",
                         "achieved": proj["kernel"]["TFLOPs"], "peak": MFMA_BF16_PEAK_TFS,
                         "unit": "TFLOP/s", "frac": proj["kernel"]["mfma_bf16_peak_frac"],
                         "traffic": measured_projection_traffic(),
                         "algorithmic_flops_per_launch": proj["kernel"]["algorithmic_flops"],
                         "avg_launch_ms": proj["kernel"]["kernel_ms"]},
            "out_roofline": {"bound": "mfma",
                             "kernel": "output projection GEMM (k_proj, one output block), "
                                       "proj_32k output side",
                             "achieved": proj["out_kernel"]["TFLOPs"], "peak": MFMA_BF16_PEAK_TFS,
                             "unit": "TFLOP/s", "frac": proj["out_kernel"]["mfma_bf16_peak_frac"],
                             "traffic": measured_projection_traffic("out"),
                             "algorithmic_flops_per_launch": proj["out_kernel"]["algorithmic_flops"],
                             "avg_launch_ms": proj["out_kernel"]["kernel_ms"]},
            **proj},
        "features_given_prefill": None if feat is None else features_given_summary(feat, main_name),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
