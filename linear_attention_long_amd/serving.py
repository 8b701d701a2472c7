"""Driving the serving calls of liblinattn for a set of requests.

Each request has a token stream (pre-activation q, k, v and, when gated, the
gate input x; the first `prompt` tokens are its prompt) and owns one row of a
state pool.  Each step, la_schedule_step picks the work (every decoding
request one token, prompts in chunks under the token budget), this module
packs those rows in that order, and la_serve_step runs the decode part and then
the prefill chunks (on one stream, or on two).  Only data movement happens here (gathering
the step's rows, scattering the outputs); every computation runs in the
library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import api


@dataclass
class Request:
    q: torch.Tensor            # [tokens, H, d] on the GPU
    k: torch.Tensor
    v: torch.Tensor
    prompt: int                # prompt tokens; the rest are decoded one per step
    x: torch.Tensor | None = None   # [tokens, H*d] gate input, or None
    slot: int = 0              # row in the state pool
    done: int = 0              # tokens processed so far
    out: list = field(default_factory=list)   # per-step output rows (on the GPU)

    @property
    def tokens(self) -> int:
        return self.q.shape[0]


def run(requests, state_pool, *, z_pool=None, w=None, normalized=False, max_batched_tokens=32768,
        out_dtype=torch.float32, two_streams=False, decode_stream=None, prefill_stream=None,
        on_step=None):
    """Process every request's whole token stream.  Returns the number of
    steps; each request's outputs end up in `torch.cat(req.out)`.  on_step,
    if given, is called with (step index, la_step_t) before each step.

    By default both parts of a step go on the current stream, decode tokens
    first: on MI355X that finishes the step sooner than two concurrent
    streams (the prefill chunk's workgroups fill every compute unit, so the
    decode kernel gains nothing from running beside them and is slowed by
    them).  two_streams=True (or passing the streams) runs them on two."""
    dev = state_pool.device
    if two_streams or decode_stream is not None or prefill_stream is not None:
        s_dec = decode_stream or torch.cuda.Stream(device=dev)
        s_pre = prefill_stream or torch.cuda.Stream(device=dev)
    else:
        s_dec = s_pre = torch.cuda.current_stream(dev)
    gated = requests[0].x is not None if requests else False
    nsteps = 0
    while True:
        live = [r for r in requests if r.done < r.tokens]
        if not live:
            return nsteps
        remaining = [max(0, r.prompt - r.done) for r in live]
        order, chunk, st = api.la_schedule_step(remaining, max_batched_tokens)
        if on_step:
            on_step(nsteps, st)
        spans = [(live[i], c) for i, c in zip(order, chunk)]
        cat = lambda name: torch.cat([getattr(r, name)[r.done:r.done + c] for r, c in spans])
        q, k, v = cat("q"), cat("k"), cat("v")
        x = cat("x") if gated else None
        nd = st.num_decode
        slots = torch.tensor([r.slot for r, _ in spans], dtype=torch.int32, device=dev)
        cu = torch.tensor([0] + [c for _, c in spans[nd:]], dtype=torch.int64).cumsum(0)
        cu = cu.to(torch.int32).to(dev)
        cur = torch.cuda.current_stream(dev)
        split = not (s_dec == cur and s_pre == cur)
        if split:
            s_dec.wait_stream(cur)
            s_pre.wait_stream(cur)
        out = api.la_serve_step(q, k, v, state_pool, slots[:nd], cu, slots[nd:],
                                max(1, st.max_chunk), x=x, w=w, z_pool=z_pool,
                                normalized=normalized, out_dtype=out_dtype,
                                decode_stream=s_dec, prefill_stream=s_pre)
        if split:
            cur.wait_stream(s_dec)
            cur.wait_stream(s_pre)
            # keep the step's inputs alive until both streams are done with them
            for t in (q, k, v, x, slots, cu, out):
                if t is not None:
                    t.record_stream(s_dec)
                    t.record_stream(s_pre)
        row = 0
        for r, c in spans:
            r.out.append(out[row:row + c])
            r.done += c
            row += c
        nsteps += 1
