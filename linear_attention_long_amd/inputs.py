"""Seeded synthetic inputs for the linear-attention path.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle take their inputs
from here.

Recipe (every workload):
  * a torch ``Generator`` seeded with ``seed * 1000 + index`` per tensor, in
    the fixed order q=0, k=1, v=2, x=3, state=4, z=5 (decode steps use
    index 100 + step);
  * values drawn as fp32 standard normals, multiplied by the workload's
    scale in fp32, then rounded to the input dtype (bf16 rounding is
    round-to-nearest-even, torch's ``.to(torch.bfloat16)``);
  * small workloads are drawn on the CPU; the 1M-token and packed workloads
    are drawn on the GPU (``device="cuda"``) because CPU generation of 4e9
    normals takes minutes.  The device is part of the recipe: the same seed
    gives different values on CPU and GPU.
  * variable lengths: numpy ``PCG64`` seeded with ``seed``, lengths
    ``round(exp(U(ln 1024, ln 131072)))`` drawn until their sum reaches the
    target; the last one is clipped to the remainder.
  * projection workloads (kind "proj"): the layer input hidden [T, K] ~
    N(0,1) (index 0) and the weight [4F, K] ~ N(0, 1/K) (index 1), rows
    [W_q; W_k; W_v; W_g], both bf16, so the projections have unit spread.
    The pages give no hidden width; K = 6144 (the bench's reading).
  * softmax-layer workloads (kind "softmax"): q [T, H, d], k and v
    [T, Hkv, d], N(0,1) in bf16 (unit-spread scores after the 1/sqrt(d)
    scale), index order q=0, k=1, v=2; packed lengths as above, drawn with
    the seed of the linear-attention workload of the same packing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "varlen" | "decode" | "serve"
    seed: int
    H: int
    d: int
    dtype: str           # "f32" | "bf16"
    T: int = 0           # prefill: tokens per sequence
    batch: int = 1       # prefill: sequences
    total_T: int = 0     # varlen: packed tokens; serve: the step's token budget
    N: int = 0           # decode / serve: decoding sequences
    steps: int = 0       # decode: steps
    scale: float = 1.0   # multiplier of the N(0,1) q, k, v draws
    block: int = 64
    gated: bool = False
    normalized: bool = False
    state_std: float = 0.0
    gen_device: str = "cpu"
    note: str = ""
    extra: dict = field(default_factory=dict)


INV_SQRT128 = 1.0 / math.sqrt(128.0)

WORKLOADS = {
    # tiny fp32 case the oracle finishes in well under a second
    "tiny_f32": Workload("tiny_f32", "prefill", 1001, H=2, d=64, dtype="f32", T=1024,
                         block=64, note="fp32, B=1 T=1024 H=2 d=64, ungated"),
    # bf16 prefill, 32K tokens, gated
    "prefill_32k": Workload("prefill_32k", "prefill", 1002, H=8, d=128, dtype="bf16",
                            T=32768, scale=INV_SQRT128, gated=True,
                            note="bf16, B=1 T=32768 H=8 d=128, RMSNorm*sigmoid gate"),
    # long-context prefill: one GPU's 8-head share of a 64-head layer
    "prefill_1m": Workload("prefill_1m", "prefill", 1003, H=8, d=128, dtype="bf16",
                           T=1048576, scale=INV_SQRT128, gated=True, gen_device="cuda",
                           note="bf16, B=1 T=1048576 H=8 d=128, RMSNorm*sigmoid gate"),
    # the pages' 4M-token inference context, same recipe (timing only)
    "prefill_4m": Workload("prefill_4m", "prefill", 1007, H=8, d=128, dtype="bf16",
                           T=4194304, scale=INV_SQRT128, gated=True, gen_device="cuda",
                           note="bf16, B=1 T=4194304 H=8 d=128, RMSNorm*sigmoid gate"),
    # packed variable-length batch
    "varlen_512k": Workload("varlen_512k", "varlen", 1004, H=8, d=128, dtype="bf16",
                            total_T=524288, scale=INV_SQRT128, gated=True, gen_device="cuda",
                            note="bf16 packed, lengths log-uniform in [1K,128K], sum 524288"),
    # decode: 64 sequences x 64 heads, 1000 steps
    "decode_64x64": Workload("decode_64x64", "decode", 1005, H=64, d=128, dtype="bf16",
                             N=64, steps=1000, state_std=0.01, gen_device="cuda",
                             note="decode, N=64 H=64 d=128, fp32 state N(0,0.01)"),
    # one serving step under a 32768-token budget: 64 decoding sequences (one
    # token each) and 32704 tokens of one prompt's chunk, all continuing from
    # fp32 states in a pool
    "serve_mixed_32k": Workload("serve_mixed_32k", "serve", 1006, H=8, d=128, dtype="bf16",
                                N=64, total_T=32768, scale=INV_SQRT128, gated=True,
                                state_std=0.01, gen_device="cuda",
                                note="serving step, 64 decode tokens + a 32704-token prompt "
                                     "chunk, H=8 d=128, gated, state pool N(0,0.01)"),
    # the layer's input projection for one GPU's 8 heads (F = 1024 features
    # each of q, k, v and the gate) from a 6144-wide layer input
    "proj_32k": Workload("proj_32k", "proj", 1011, H=8, d=128, dtype="bf16", T=32768,
                         gen_device="cuda", extra={"K": 6144},
                         note="input projection, bf16 hidden [32768, 6144] x weight "
                              "[4096, 6144] -> q, k, v (SiLU) and gate pre-activation"),
    "proj_1m": Workload("proj_1m", "proj", 1012, H=8, d=128, dtype="bf16", T=1048576,
                        gen_device="cuda", extra={"K": 6144},
                        note="input projection of the 1M-token sequence, hidden "
                             "[1048576, 6144] x weight [4096, 6144]"),
    # the softmax attention layer of the hybrid model on the same shapes:
    # one GPU's 8 heads, rotary embedding on half of d = 128, the
    # long-context base 1e7, Hkv = H
    "softmax_32k": Workload("softmax_32k", "softmax", 1008, H=8, d=128, dtype="bf16", T=32768,
                            extra={"Hkv": 8, "rotary_dim": 64, "rope_base": 1e7},
                            note="softmax layer, bf16, T=32768 H=8 Hkv=8 d=128, RoPE on 64 "
                                 "dims, base 1e7"),
    "softmax_varlen_512k": Workload("softmax_varlen_512k", "softmax", 1009, H=8, d=128,
                                    dtype="bf16", total_T=524288, gen_device="cuda",
                                    extra={"Hkv": 8, "rotary_dim": 64, "rope_base": 1e7,
                                           "length_seed": 1004},
                                    note="softmax layer, bf16 packed, lengths of varlen_512k, "
                                         "H=8 Hkv=8 d=128, RoPE on 64 dims, base 1e7"),
    "softmax_1m": Workload("softmax_1m", "softmax", 1010, H=8, d=128, dtype="bf16", T=1048576,
                           gen_device="cuda",
                           extra={"Hkv": 8, "rotary_dim": 64, "rope_base": 1e7},
                           note="softmax layer, bf16, T=1048576 H=8 Hkv=8 d=128, RoPE on 64 "
                                "dims, base 1e7"),
}


def _gen(seed: int, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(index))
    return g


def normal(shape, seed: int, index: int, scale: float = 1.0, dtype=torch.float32,
           device="cpu") -> torch.Tensor:
    """N(0,1) * scale drawn in fp32 on ``device`` with a per-tensor seed, then
    rounded to ``dtype``."""
    g = _gen(seed, index, device)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if scale != 1.0:
        t.mul_(float(scale))
    return t.to(dtype)


def varlen_lengths(seed: int, total: int, lo: int = 1024, hi: int = 131072) -> list:
    """Lengths round(exp(U(ln lo, ln hi))) until they sum to ``total``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out, acc = [], 0
    while acc < total:
        L = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = max(1, min(L, total - acc))
        out.append(L)
        acc += L
    return out


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def prefill_inputs(w: Workload, T: int | None = None, batch: int | None = None,
                   device: str | None = None, with_gate: bool | None = None):
    """q, k, v [batch, T, H, d] and x [batch, T, H*d] (or None) for a
    prefill workload; ``T``/``batch`` override the workload's sizes."""
    T = w.T if T is None else T
    batch = w.batch if batch is None else batch
    dev = w.gen_device if device is None else device
    dt = DTYPES[w.dtype]
    shape = (batch, T, w.H, w.d)
    q = normal(shape, w.seed, 0, w.scale, dt, dev)
    k = normal(shape, w.seed, 1, w.scale, dt, dev)
    v = normal(shape, w.seed, 2, w.scale, dt, dev)
    gate = w.gated if with_gate is None else with_gate
    x = normal((batch, T, w.H * w.d), w.seed, 3, 1.0, dt, dev) if gate else None
    return q, k, v, x


def varlen_inputs(w: Workload, total_T: int | None = None, device: str | None = None):
    """Packed q, k, v [total_T, H, d], x [total_T, H*d] and cu_seqlens (int32,
    CPU) for a varlen workload."""
    total = w.total_T if total_T is None else total_T
    dev = w.gen_device if device is None else device
    dt = DTYPES[w.dtype]
    lengths = varlen_lengths(w.seed, total)
    cu = cu_from_lengths(lengths)
    shape = (total, w.H, w.d)
    q = normal(shape, w.seed, 0, w.scale, dt, dev)
    k = normal(shape, w.seed, 1, w.scale, dt, dev)
    v = normal(shape, w.seed, 2, w.scale, dt, dev)
    x = normal((total, w.H * w.d), w.seed, 3, 1.0, dt, dev) if w.gated else None
    return q, k, v, x, cu


def serve_inputs(w: Workload, device: str | None = None):
    """One serving step: packed q, k, v [total_T, H, d] and x [total_T, H*d]
    (rows [0, N) are the decode tokens, the rest one prompt chunk) and the
    fp32 state pool [N + 1, H, d, d] (row N belongs to the prompt)."""
    dev = w.gen_device if device is None else device
    dt = DTYPES[w.dtype]
    shape = (w.total_T, w.H, w.d)
    q = normal(shape, w.seed, 0, w.scale, dt, dev)
    k = normal(shape, w.seed, 1, w.scale, dt, dev)
    v = normal(shape, w.seed, 2, w.scale, dt, dev)
    x = normal((w.total_T, w.H * w.d), w.seed, 3, 1.0, dt, dev) if w.gated else None
    pool = normal((w.N + 1, w.H, w.d, w.d), w.seed, 4, w.state_std, torch.float32, dev)
    return q, k, v, x, pool


def decode_state(w: Workload, N: int | None = None, H: int | None = None, device=None):
    """Initial fp32 state S [N, H, d, d] and normaliser z [N, H, d], N(0, std)."""
    N = w.N if N is None else N
    H = w.H if H is None else H
    dev = w.gen_device if device is None else device
    S = normal((N, H, w.d, w.d), w.seed, 4, w.state_std, torch.float32, dev)
    z = normal((N, H, w.d), w.seed, 5, w.state_std, torch.float32, dev)
    return S, z


def decode_token(w: Workload, step: int, N: int | None = None, H: int | None = None,
                 device=None):
    """Pre-activation q, k, v [N, H, d] of decode step ``step``."""
    N = w.N if N is None else N
    H = w.H if H is None else H
    dev = w.gen_device if device is None else device
    dt = DTYPES[w.dtype]
    g = _gen(w.seed, 100 + step, dev)
    t = torch.randn((3, N, H, w.d), generator=g, dtype=torch.float32, device=dev)
    if w.scale != 1.0:
        t.mul_(float(w.scale))
    t = t.to(dt)
    return t[0], t[1], t[2]


def softmax_inputs(w: Workload, device: str | None = None, Hkv: int | None = None):
    """q [total, H, d], k and v [total, Hkv, d] (bf16) and cu_seqlens (int32,
    CPU) of a softmax-layer workload: one sequence of w.T tokens, or the
    packed lengths of ``extra["length_seed"]`` summing to w.total_T."""
    dev = w.gen_device if device is None else device
    dt = DTYPES[w.dtype]
    Hkv = w.extra.get("Hkv", w.H) if Hkv is None else Hkv
    if w.total_T:
        total = w.total_T
        cu = cu_from_lengths(varlen_lengths(w.extra.get("length_seed", w.seed), total))
    else:
        total = w.T
        cu = torch.tensor([0, total], dtype=torch.int32)
    q = normal((total, w.H, w.d), w.seed, 0, w.scale, dt, dev)
    k = normal((total, Hkv, w.d), w.seed, 1, w.scale, dt, dev)
    v = normal((total, Hkv, w.d), w.seed, 2, w.scale, dt, dev)
    return q, k, v, cu


def projection_inputs(w: Workload, T: int | None = None, device=None):
    """hidden [T, K] ~ N(0,1) and weight [4F, K] ~ N(0, 1/K), both bf16."""
    T = w.T if T is None else T
    K = w.extra["K"]
    F = w.H * w.d
    dev = w.gen_device if device is None else device
    hidden = normal((T, K), w.seed, 0, 1.0, torch.bfloat16, dev)
    weight = normal((4 * F, K), w.seed, 1, 1.0 / math.sqrt(K), torch.bfloat16, dev)
    return hidden, weight


def out_projection_inputs(w: Workload, T: int | None = None, device=None):
    """The output projection's operands for the same layer: y [T, F] ~ N(0,1)
    (a stand-in for the gated attention output, which the RMSNorm leaves at
    unit scale) and W_o [K, F] ~ N(0, 1/F) (hidden width K = the input
    projection's), both bf16."""
    T = w.T if T is None else T
    K = w.extra["K"]
    F = w.H * w.d
    dev = w.gen_device if device is None else device
    y = normal((T, F), w.seed, 2, 1.0, torch.bfloat16, dev)
    wo = normal((K, F), w.seed, 3, 1.0 / math.sqrt(F), torch.bfloat16, dev)
    return y, wo
