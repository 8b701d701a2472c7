"""Causal linear attention (Lightning Attention forward) on AMD MI355X.

The computation runs in the HIP library ``liblinattn.so`` (C ABI in
include/la.h, and include/la_softmax.h for the hybrid model's softmax
attention layer); this package holds its Python binding (:mod:`.api`), the build
step (:mod:`.build`) and the seeded input generator (:mod:`.inputs`).
"""
from __future__ import annotations

__all__ = ["la_prefill", "la_prefill_varlen", "la_decode_step", "prefill", "prefill_varlen",
           "decode_step", "la_softmax_attention_varlen"]


def __getattr__(name):
    if name in __all__:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
