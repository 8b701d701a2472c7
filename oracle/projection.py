"""CPU oracle of the input and output projections of a lightning-attention
layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares nothing with the HIP library.

Page "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1, writes the
layer as Q, K, V = SiLU(X) (the projection of the layer input X by its
weights is implied: Q = SiLU(X W_q), likewise K and V), the linear
attention Y = Q (K^T V), and the output RMSNorm(Y) * sigmoid(X) with the
gate taken from X through a projection of its own.  For one GPU's share of
the heads (H heads of head dim d, F = H * d features per token) the
projection is one product with four column blocks:

    P = hidden @ W^T,  W = [W_q; W_k; W_v; W_g]   (W: [4F, K], rows are output features)
    q, k, v = SiLU(P[:, 0:F]), SiLU(P[:, F:2F]), SiLU(P[:, 2F:3F])   (featurize)
    x_gate  = P[:, 3F:4F]                                            (gate pre-activation)

With ``featurize=False`` the first three blocks are returned unactivated
(pre-activations for a path that applies SiLU itself).  Everything is fp64:
numpy's matmul on the exactly widened inputs, SiLU(x) = x / (1 + exp(-x)).
The output projection maps the gated attention output back to the hidden
width: page "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南",
FAQ Q5 (fine-tuning), names the attention layer's four projection matrices
Q, K, V and O.  For one GPU's heads (its F = H * d columns of the gated
output) the product with the matching columns of W_o is that GPU's partial
sum of the layer output:

    out = y @ W_o^T,   y: [T, F] gated output,  W_o: [N, F]  (row n = hidden feature n)

and the partial sums of the GPUs holding the other heads add up to the
whole product (the identity ``test_out_projection_column_split_sums_to_the_whole``
pins).

The pins (``tests/test_oracle_projection_pins.py``) check both against
pure-Python triple loops, closed forms for selection and constant weights,
and the composition with the pinned path oracle.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if hasattr(a, "detach"):
        import torch

        a = a.detach().to("cpu")
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.to(torch.float32)
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def silu(x):
    return x / (1.0 + np.exp(-x))


def project(hidden, weight, F, featurize=True, rows=None):
    """hidden [T, K], weight [4F, K] (any float dtype, widened exactly).
    Returns (q, k, v, x_gate), each [T, F] fp64 (or [len(rows), F] for the
    listed token rows)."""
    h = _f64(hidden)
    if rows is not None:
        h = h[np.asarray(rows, dtype=np.int64)]
    W = _f64(weight)
    if W.shape[0] != 4 * F or W.shape[1] != h.shape[1]:
        raise ValueError("weight must be [4F, K] with K = hidden's width")
    P = h @ W.T
    blocks = [P[:, i * F:(i + 1) * F] for i in range(4)]
    if featurize:
        blocks = [silu(b) for b in blocks[:3]] + [blocks[3]]
    return tuple(np.ascontiguousarray(b) for b in blocks)


def out_project(y, weight, rows=None):
    """y [T, F] (the gated attention output), weight [N, F] (any float dtype,
    widened exactly).  Returns y @ weight^T, [T, N] fp64 (or [len(rows), N]
    for the listed token rows)."""
    a = _f64(y)
    if rows is not None:
        a = a[np.asarray(rows, dtype=np.int64)]
    W = _f64(weight)
    if W.ndim != 2 or a.ndim != 2 or W.shape[1] != a.shape[1]:
        raise ValueError("weight must be [N, F] with F = y's width")
    return np.ascontiguousarray(a @ W.T)
