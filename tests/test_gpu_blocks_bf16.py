"""bf16 inputs in the default (SiLU) mode at the pages' block sizes.

The deployment page (xdnf.cn, on MoE memory under long context, section 3)
runs lightning attention in blocks of 256 tokens and pads a partial tail
block to the nearest of 32, 64 or 128 rows.  The block size only changes the
fp32 rounding order (the blocked form is a reassociation of the causal sum),
so every block must agree with the oracle.  With bf16 inputs, blocks of 128
and 256 (and head dim 64 at any block) run on the fp32 vector kernel, which
evaluates the blocked form at exactly that block in 32-row sub-tiles: a tail
of r rows is processed as ceil(r / 32) sub-tiles, i.e. padded to a multiple
of 32 no larger than the pages' pad (zeros add nothing, SiLU(0) = 0).

Tails are chosen in each of the pages' pad classes for a 256-token block,
r in (0, 32], (32, 64], (64, 128] and (128, 256), and the like for 128.
Every element of the output and the final state is compared with the oracle
at 1e-2 of rms (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

from linear_attention_long_amd import _lib, api, inputs
from oracle import oracle as O
from tests._util import banner, np64, randn, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda"


def bf16_inputs(T, H, d, seed, gated, shift=0.0):
    s = 1.0 / np.sqrt(d)
    q, k = (randn((T, H, d), seed + i, s if not shift else 0.5, shift, dtype=torch.bfloat16)
            for i in range(2))
    v = randn((T, H, d), seed + 2, s, dtype=torch.bfloat16)
    x = randn((T, H * d), seed + 3, dtype=torch.bfloat16) if gated else None
    return q, k, v, x


# (block, tail rows r): each of the pad classes (0,32], (32,64], (64,128],
# (128,256) for block 256, and (0,32], (32,64], (64,128) for block 128
TAILS = [(256, 1), (256, 32), (256, 50), (256, 64), (256, 65), (256, 100), (256, 128),
         (256, 129), (256, 200), (256, 255), (256, 0),
         (128, 17), (128, 32), (128, 40), (128, 64), (128, 100), (128, 127), (128, 0)]


@pytest.mark.parametrize("block,r", TAILS)
def test_bf16_d128_block_tail_classes_gated(block, r):
    T, H, d = 2 * block + r, 4, 128
    banner("bf16 d=128 block %d tail %d gated (T=%d)" % (block, r, T))
    plan = _lib.plan(False, 1, T, T, H, d, _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32,
                     _lib.options(block_size=block, gated=True))
    assert plan.block_size == block
    q, k, v, x = bf16_inputs(T, H, d, 500 + r, True)
    out, S, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), block_size=block)
    ref, Sref, _ = O.forward(q, k, v, x, gated=True)
    e, es = rel_err(np64(out), ref), rel_err(np64(S), Sref[0])   # [T, H, d] in: S is [H, d, d]
    assert e <= TOL and es <= TOL, (e, es)


@pytest.mark.parametrize("block,r", [(128, 100), (256, 50), (256, 200), (256, 255)])
def test_bf16_d128_block_tail_normalized(block, r):
    T, H, d = 3 * block + r, 2, 128
    banner("bf16 d=128 block %d tail %d normalised" % (block, r))
    q, k, v, _ = bf16_inputs(T, H, d, 600 + r, False, shift=1.0)
    z0 = torch.ones((1, H, d))
    out, S, z = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), None, None, None, z0.to(DEV),
                               normalized=True, block_size=block)
    ref, Sref, zref = O.forward(q, k, v, z_in=z0, normalized=True)
    assert rel_err(np64(out), ref) <= TOL
    assert rel_err(np64(S), Sref[0]) <= TOL
    assert rel_err(np64(z), zref[0]) <= 1e-4


@pytest.mark.parametrize("block", [128, 256])
@pytest.mark.parametrize("chunk", [256, 512, 1024])
def test_bf16_d128_block_chunked_with_state(block, chunk):
    """Chunks of 256-1024 tokens over blocks of 128/256 (chunk boundaries at,
    and inside, block boundaries), a carried state_in and two sequences."""
    Bt, T, H, d = 2, 2100, 4, 128
    banner("bf16 d=128 block %d chunk %d with state" % (block, chunk))
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((Bt, T, H, d), 700 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((Bt, T, H * d), 703, dtype=torch.bfloat16)
    S0 = randn((Bt, H, d, d), 704, 0.05)
    out, S, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), None, S0.to(DEV),
                               block_size=block, chunk_tokens=chunk)
    for b in range(Bt):
        ref, Sref, _ = O.forward(q[b], k[b], v[b], x[b], state_in=S0[b:b + 1], gated=True)
        assert rel_err(np64(out[b]), ref) <= TOL
        assert rel_err(np64(S[b]), Sref[0]) <= TOL


@pytest.mark.parametrize("block", [32, 64, 128, 256])
@pytest.mark.parametrize("T,gated", [(1, True), (333, True), (1000, False), (1000, True)])
def test_bf16_d64(block, T, gated):
    H, d = 4, 64
    banner("bf16 d=64 block %d T=%d gated=%s" % (block, T, gated))
    q, k, v, x = bf16_inputs(T, H, d, 800 + T, gated)
    out, S, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), None if x is None else x.to(DEV),
                               block_size=block)
    ref, Sref, _ = O.forward(q, k, v, x, gated=gated)
    assert rel_err(np64(out), ref) <= TOL
    assert rel_err(np64(S), Sref[0]) <= TOL


def test_bf16_d64_varlen_and_decode():
    """Head dim 64, bf16: a packed batch (empty, one-token and multi-block
    sequences) at block 256, and decode steps continuing from its states."""
    H, d = 4, 64
    lengths = [300, 0, 1, 700, 257]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    q, k, v, x = bf16_inputs(int(cu[-1]), H, d, 900, True)
    cud = torch.tensor(cu, dtype=torch.int32, device=DEV)
    out, S, _ = api.la_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cud, 700, x.to(DEV),
                                      block_size=256)
    ref, Sref, _ = O.forward(q, k, v, x, cu_seqlens=cu, gated=True)
    assert rel_err(np64(out), ref) <= TOL
    assert rel_err(np64(S), Sref) <= TOL
    qd, kd, vd, _ = bf16_inputs(len(lengths), H, d, 910, False)
    Sd = S.clone()
    y = api.la_decode_step(qd.to(DEV), kd.to(DEV), vd.to(DEV), Sd)
    yref, Snew, _ = O.decode_step(qd, kd, vd, Sref)
    assert rel_err(np64(y), yref.reshape(len(lengths), H * d)) <= TOL
    assert rel_err(np64(Sd), Snew) <= TOL


def test_prefill_32k_workload_block_256():
    """The 32K-token workload at its configured block of 256 tokens (bf16,
    T=32768, H=8, d=128, gated): every output and the final state."""
    w = inputs.WORKLOADS["prefill_32k"]
    banner("prefill_32k workload at block 256")
    q, k, v, x = inputs.prefill_inputs(w)
    out, S, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), block_size=256)
    torch.cuda.synchronize()
    ref, Sref, _ = O.forward(q[0], k[0], v[0], x[0], gated=True)
    e_out, e_S = rel_err(np64(out[0]), ref), rel_err(np64(S[0]), Sref[0])
    print("prefill_32k block 256: rel err out %.3e state %.3e" % (e_out, e_S))
    assert e_out <= TOL and e_S <= TOL
