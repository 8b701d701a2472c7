"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Tolerances (max|err| / rms(ref), over every element compared):
  * fp32 inputs: 1e-5 -- fp32 arithmetic throughout;
  * bf16 inputs: 1e-2 -- bf16 matrix-core operands (hi/lo split on the
    inter-block and state products), fp32 accumulation, fp32 output.
The oracle runs in fp64 on the same (bf16- or fp32-valued) inputs.
"""
import numpy as np
import pytest
import torch

from linear_attention_long_amd import _lib, api, inputs
from oracle import oracle as O
from tests._util import banner, np64, randn, rel_err

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 1e-2
DEV = "cuda"


def run_prefill(q, k, v, x=None, **kw):
    out, S, z = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV),
                               None if x is None else x.to(DEV), **kw)
    torch.cuda.synchronize()
    return out, S, z


def oracle_forward(q, k, v, x=None, state_in=None, z_in=None, normalized=False, norm_group=0):
    """Oracle on [Bt, T, H, d] inputs -> out [Bt, T, H*d], S [Bt, H, d, d], z."""
    Bt, T, H, d = q.shape
    outs, Ss, zs = [], [], []
    for b in range(Bt):
        o, S, z = O.forward(q[b], k[b], v[b], None if x is None else x[b], None,
                            state_in=None if state_in is None else state_in[b:b + 1],
                            z_in=None if z_in is None else z_in[b:b + 1],
                            normalized=normalized, gated=x is not None, norm_group=norm_group)
        outs.append(o)
        Ss.append(S[0])
        zs.append(z[0])
    return np.stack(outs), np.stack(Ss), np.stack(zs)


# ---------------------------------------------------------------- fp32 path --

def test_tiny_f32_workload():
    """fp32, B=1 T=1024 H=2 d=64, block 64, ungated, unnormalised."""
    w = inputs.WORKLOADS["tiny_f32"]
    banner("tiny_f32 workload")
    q, k, v, _ = inputs.prefill_inputs(w)
    out, S, _ = run_prefill(q, k, v, block_size=w.block)
    ref, Sref, _ = oracle_forward(q, k, v)
    assert rel_err(np64(out), ref.reshape(out.shape)) <= TOL_F32
    assert rel_err(np64(S), Sref) <= TOL_F32


@pytest.mark.parametrize("block", [32, 64, 128, 256])
@pytest.mark.parametrize("T,chunk", [(1000, 0), (1000, 256), (1, 0), (33, 0), (300, 64)])
def test_f32_block_sizes_and_tails(block, T, chunk):
    banner("f32 block=%d T=%d chunk=%d" % (block, T, chunk))
    H, d = 2, 64
    q, k, v = (randn((1, T, H, d), 10 + i) for i in range(3))
    out, S, _ = run_prefill(q, k, v, block_size=block, chunk_tokens=chunk)
    ref, Sref, _ = oracle_forward(q, k, v)
    assert rel_err(np64(out), ref.reshape(out.shape)) <= TOL_F32
    assert rel_err(np64(S), Sref) <= TOL_F32


def test_f32_d128_gated_normalized_with_state():
    banner("f32 d=128 gated normalised with state")
    Bt, T, H, d = 2, 200, 2, 128
    q, k = (randn((Bt, T, H, d), 20 + i, 0.5, 1.0) for i in range(2))
    v = randn((Bt, T, H, d), 22)
    x = randn((Bt, T, H * d), 23)
    S0 = randn((Bt, H, d, d), 24, 0.01).abs()
    z0 = randn((Bt, H, d), 25, 0.1).abs() + 1.0
    out, S, z = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), None, S0.to(DEV),
                               z0.to(DEV), normalized=True, chunk_tokens=64)
    ref, Sref, zref = oracle_forward(q, k, v, x, S0, z0, normalized=True)
    assert rel_err(np64(out), ref) <= TOL_F32
    assert rel_err(np64(S), Sref) <= TOL_F32
    assert rel_err(np64(z), zref) <= TOL_F32


# ---------------------------------------------------- bf16 matrix-core path --

@pytest.mark.parametrize("T", [1, 17, 32, 33, 64, 100, 1000, 2085])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("block", [32, 64])
def test_bf16_short_sequences(T, gated, block):
    banner("bf16 T=%d gated=%s block=%d" % (T, gated, block))
    H, d = 2, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 30 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((1, T, H * d), 33, dtype=torch.bfloat16) if gated else None
    out, S, _ = run_prefill(q, k, v, x, block_size=block)
    ref, Sref, _ = oracle_forward(q, k, v, x)
    assert rel_err(np64(out), ref) <= TOL_BF16
    assert rel_err(np64(S), Sref) <= TOL_BF16


@pytest.mark.parametrize("chunk", [64, 1024])
@pytest.mark.parametrize("block", [32, 64])
def test_bf16_chunked_with_state_in(chunk, block):
    banner("bf16 chunked chunk=%d block=%d" % (chunk, block))
    Bt, T, H, d = 2, 3000, 4, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((Bt, T, H, d), 40 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((Bt, T, H * d), 43, dtype=torch.bfloat16)
    S0 = randn((Bt, H, d, d), 44, 0.05)
    out, S, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), None, S0.to(DEV),
                               chunk_tokens=chunk, block_size=block)
    ref, Sref, _ = oracle_forward(q, k, v, x, S0)
    assert rel_err(np64(out), ref) <= TOL_BF16
    assert rel_err(np64(S), Sref) <= TOL_BF16


@pytest.mark.parametrize("block", [32, 64])
def test_bf16_normalized(block):
    banner("bf16 normalised block=%d" % block)
    Bt, T, H, d = 1, 1500, 2, 128
    q, k = (randn((Bt, T, H, d), 50 + i, 0.5, 1.0, dtype=torch.bfloat16) for i in range(2))
    v = randn((Bt, T, H, d), 52, dtype=torch.bfloat16)
    z0 = torch.ones((Bt, H, d))
    for chunk in (0, 512):
        out, S, z = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), None, None, None, z0.to(DEV),
                                   normalized=True, chunk_tokens=chunk, block_size=block)
        ref, Sref, zref = oracle_forward(q, k, v, None, None, z0, normalized=True)
        assert rel_err(np64(out), ref.reshape(out.shape)) <= TOL_BF16
        assert rel_err(np64(z), zref) <= 1e-4


def test_bf16_out_dtype_and_weight():
    banner("bf16 output, rms weight, per-head norm group")
    T, H, d = 700, 4, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 60 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((1, T, H * d), 63, dtype=torch.bfloat16)
    w = randn((H * d,), 64, 0.2, 1.0)
    for group in (0, d):
        out, _, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), w.to(DEV),
                                   norm_group=group, out_dtype=torch.float32)
        ref, _, _ = O.forward(q[0], k[0], v[0], x[0], w, gated=True, norm_group=group)
        assert rel_err(np64(out[0]), ref) <= TOL_BF16
        outb, _, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), w.to(DEV),
                                    norm_group=group, out_dtype=torch.bfloat16)
        # bf16 storage adds up to half an ulp (<= 2^-8 of |value|, 8 significant bits)
        # on top of the fp32-output error bound
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(np64(outb[0]) - ref)
        assert (err <= 2.0 ** -8 * np.abs(ref) + TOL_BF16 * rms).all()


def test_prefill_32k_workload():
    """bf16, T=32768, H=8, d=128, gated: every output and the final state."""
    w = inputs.WORKLOADS["prefill_32k"]
    banner("prefill_32k workload")
    q, k, v, x = inputs.prefill_inputs(w)
    out, S, _ = run_prefill(q, k, v, x)
    ref, Sref, _ = oracle_forward(q, k, v, x)
    e_out, e_S = rel_err(np64(out), ref), rel_err(np64(S), Sref)
    print("prefill_32k rel err out %.3e state %.3e" % (e_out, e_S))
    assert e_out <= TOL_BF16 and e_S <= TOL_BF16


@pytest.mark.parametrize("gated,block", [(False, 32), (False, 64), (True, 32)])
def test_bf16_split_precision_canary(gated, block):
    """The matrix-core path splits every operand into bf16 hi + lo (about 16
    significant bits), so its error sits near 1e-5 .. 1e-4 of rms here.  A
    split that lost its low part would err by ~1e-3 and still pass the 1e-2
    tolerance; this bound (5e-4, an implementation check, not the tolerance)
    catches that."""
    banner("bf16 split precision canary gated=%s block=%d" % (gated, block))
    T, H, d = 1000, 2, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 180 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((1, T, H * d), 183, dtype=torch.bfloat16) if gated else None
    out, S, _ = run_prefill(q, k, v, x, block_size=block)
    ref, Sref, _ = oracle_forward(q, k, v, x)
    e_out, e_S = rel_err(np64(out), ref), rel_err(np64(S), Sref)
    print("canary: rel err out %.3e state %.3e" % (e_out, e_S))
    assert e_out <= 5e-4 and e_S <= 5e-4


# ---------------------------------------------------------- fused gate path --
# bf16 d=128 gated calls whose (chunk, head) workgroups fit on the device at
# once run the gate inside the main pass (heads of a chunk exchange their
# per-token sums of y^2).  Each case checks that the plan fuses, then parity.

def fused_plan(varlen, num_seqs, total, max_len, H, out_dtype=_lib.LA_DTYPE_F32, **kw):
    return _lib.plan(varlen, num_seqs, total, max_len, H, 128, _lib.LA_DTYPE_BF16, out_dtype,
                     _lib.options(gated=True, **kw))


@pytest.mark.parametrize("Bt,T,H,chunk,normalized", [
    (1, 1, 1, 0, False),       # one token, one head
    (1, 31, 8, 0, False),      # ragged single block, the most heads fused
    (2, 33, 3, 0, False),      # odd head count, 32-row block + 1-row tail
    (1, 1000, 8, 0, True),     # normalised mode
    (1, 5000, 5, 512, False),  # several chunks (prefix scan) per sequence
    (2, 3001, 8, 1024, True),  # chunks + normalised + batch, ragged tail
    (1, 4096, 2, 0, False),
])
def test_fused_gate(Bt, T, H, chunk, normalized):
    banner("fused gate Bt=%d T=%d H=%d chunk=%d normalized=%s" % (Bt, T, H, chunk, normalized))
    d = 128
    plan = fused_plan(False, Bt, Bt * T, T, H, chunk_tokens=chunk, normalized=normalized)
    assert plan.fused_gate == 1, plan.kernel_names()
    if normalized:
        q, k = (randn((Bt, T, H, d), 140 + i, 0.5, 1.0, dtype=torch.bfloat16) for i in range(2))
    else:
        q, k = (randn((Bt, T, H, d), 140 + i, 1.0 / np.sqrt(d), dtype=torch.bfloat16)
                for i in range(2))
    v = randn((Bt, T, H, d), 142, dtype=torch.bfloat16)
    x = randn((Bt, T, H * d), 143, dtype=torch.bfloat16)
    S0 = randn((Bt, H, d, d), 144, 0.02)
    z0 = torch.ones((Bt, H, d)) if normalized else None
    out, S, z = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), None, S0.to(DEV),
                               None if z0 is None else z0.to(DEV), normalized=normalized,
                               chunk_tokens=chunk)
    torch.cuda.synchronize()
    ref, Sref, zref = oracle_forward(q, k, v, x, S0, z0, normalized=normalized)
    assert rel_err(np64(out), ref) <= TOL_BF16
    assert rel_err(np64(S), Sref) <= TOL_BF16
    if normalized:
        assert rel_err(np64(z), zref) <= 1e-4


def test_fused_gate_bf16_out_and_weight():
    banner("fused gate, bf16 output, rms weight")
    T, H, d = 2085, 8, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 150 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((1, T, H * d), 153, dtype=torch.bfloat16)
    w = randn((H * d,), 154, 0.2, 1.0)
    assert fused_plan(False, 1, T, T, H, _lib.LA_DTYPE_BF16).fused_gate == 1
    outb, _, _ = api.la_prefill(q.to(DEV), k.to(DEV), v.to(DEV), x.to(DEV), w.to(DEV),
                                out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, _, _ = O.forward(q[0], k[0], v[0], x[0], w, gated=True)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(np64(outb[0]) - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + TOL_BF16 * rms).all()


def test_fused_gate_varlen():
    banner("fused gate, varlen with empty sequences")
    lengths = [1, 0, 100, 64, 1500, 33, 0, 257, 4000]
    cu = inputs.cu_from_lengths(lengths)
    total, H, d = int(cu[-1]), 4, 128
    s = 1.0 / np.sqrt(d)
    for chunk in (0, 512):
        plan = fused_plan(True, len(lengths), total, max(lengths), H, chunk_tokens=chunk)
        assert plan.fused_gate == 1, plan.kernel_names()
        q, k, v = (randn((total, H, d), 160 + i, s, dtype=torch.bfloat16) for i in range(3))
        x = randn((total, H * d), 163, dtype=torch.bfloat16)
        S0 = randn((len(lengths), H, d, d), 164, 0.05)
        out, S, _ = api.la_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV),
                                          max(lengths), x.to(DEV), None, S0.to(DEV),
                                          chunk_tokens=chunk)
        torch.cuda.synchronize()
        ref, Sref, _ = O.forward(q, k, v, x, None, cu_seqlens=cu.numpy(), state_in=S0, gated=True)
        assert rel_err(np64(out), ref) <= TOL_BF16
        assert rel_err(np64(S), Sref) <= TOL_BF16
        assert torch.equal(S[1].cpu(), S0[1]) and torch.equal(S[6].cpu(), S0[6])


def test_fused_gate_varlen_device_chunking():
    """40 sequences of 50..3000 tokens, 8 heads: the fused plan's chunk length
    is searched on the device (below the worst-case bound the host sets);
    every output and final state against the oracle."""
    banner("fused gate, varlen, chunk length chosen on the device")
    rng = np.random.default_rng(190)
    lengths = rng.integers(50, 3001, size=40).tolist()
    cu = inputs.cu_from_lengths(lengths)
    total, H, d = int(cu[-1]), 8, 128
    plan = fused_plan(True, len(lengths), total, max(lengths), H)
    assert plan.fused_gate == 1 and plan.chunk_on_device == 1, plan.kernel_names()
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((total, H, d), 191 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((total, H * d), 194, dtype=torch.bfloat16)
    S0 = randn((len(lengths), H, d, d), 195, 0.05)
    out, S, _ = api.la_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths),
                                      x.to(DEV), None, S0.to(DEV))
    torch.cuda.synchronize()
    ref, Sref, _ = O.forward(q, k, v, x, None, cu_seqlens=cu.numpy(), state_in=S0, gated=True)
    e_out, e_S = rel_err(np64(out), ref), rel_err(np64(S), Sref)
    print("varlen device chunking (host bound %d tokens): rel err out %.3e state %.3e"
          % (plan.chunk_tokens, e_out, e_S))
    assert e_out <= TOL_BF16 and e_S <= TOL_BF16


@pytest.mark.parametrize("varlen", [True, False])
def test_more_sequences_than_resident_teams(varlen):
    """150 sequences with 8 heads: more teams than the device keeps resident,
    so the gate runs as its own kernel after the main pass; every output and
    final state against the oracle."""
    banner("150 sequences, varlen=%s (gate not fused)" % varlen)
    H, d = 8, 128
    rng = np.random.default_rng(321)
    lengths = rng.integers(0, 300, size=150).tolist() if varlen else [97] * 150
    cu = inputs.cu_from_lengths(lengths)
    total = int(cu[-1])
    plan = fused_plan(varlen, len(lengths), total, max(lengths), H)
    assert plan.fused_gate == 0 and plan.kernel_names()[-2:] == ["main", "gate"], plan.kernel_names()
    s_ = 1.0 / np.sqrt(d)
    q, k, v = (randn((total, H, d), 330 + i, s_, dtype=torch.bfloat16) for i in range(3))
    x = randn((total, H * d), 333, dtype=torch.bfloat16)
    S0 = randn((len(lengths), H, d, d), 334, 0.05)
    if varlen:
        out, S, _ = api.la_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths),
                                          x.to(DEV), None, S0.to(DEV))
    else:
        T = lengths[0]
        out, S, _ = api.la_prefill(q.reshape(150, T, H, d).to(DEV), k.reshape(150, T, H, d).to(DEV),
                                   v.reshape(150, T, H, d).to(DEV), x.reshape(150, T, H * d).to(DEV),
                                   None, S0.to(DEV))
        out = out.reshape(total, H * d)
    torch.cuda.synchronize()
    ref, Sref, _ = O.forward(q, k, v, x, None, cu_seqlens=cu.numpy(), state_in=S0, gated=True)
    assert rel_err(np64(out), ref) <= TOL_BF16
    assert rel_err(np64(S), Sref) <= TOL_BF16


def test_unfused_gate_when_heads_exceed_fused_limit():
    banner("gate not fused: H=9 (unfused path), parity")
    T, H, d = 700, 9, 128
    plan = fused_plan(False, 1, T, T, H)
    assert plan.fused_gate == 0 and plan.kernel_names()[-2:] == ["main", "gate"]
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 170 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((1, T, H * d), 173, dtype=torch.bfloat16)
    out, S, _ = run_prefill(q, k, v, x)
    ref, Sref, _ = oracle_forward(q, k, v, x)
    assert rel_err(np64(out), ref) <= TOL_BF16
    assert rel_err(np64(S), Sref) <= TOL_BF16


# ------------------------------------------------------------------- varlen --

@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("chunk", [0, 128])
def test_varlen_matches_oracle(dtype, d, chunk):
    banner("varlen dtype=%s d=%d chunk=%d" % (dtype, d, chunk))
    lengths = [1, 0, 100, 64, 1500, 33, 0, 257]
    cu = inputs.cu_from_lengths(lengths)
    total, H = int(cu[-1]), 2
    s = 1.0 / np.sqrt(d) if dtype == torch.bfloat16 else 1.0
    q, k, v = (randn((total, H, d), 70 + i, s, dtype=dtype) for i in range(3))
    x = randn((total, H * d), 73, dtype=dtype)
    S0 = randn((len(lengths), H, d, d), 74, 0.05)
    out, S, _ = api.la_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths),
                                      x.to(DEV), None, S0.to(DEV), chunk_tokens=chunk)
    torch.cuda.synchronize()
    ref, Sref, _ = O.forward(q, k, v, x, None, cu_seqlens=cu.numpy(), state_in=S0, gated=True)
    tol = TOL_BF16 if dtype == torch.bfloat16 else TOL_F32
    assert rel_err(np64(out), ref) <= tol
    assert rel_err(np64(S), Sref) <= tol
    # empty sequences hand their state through unchanged
    assert torch.equal(S[1].cpu(), S0[1]) and torch.equal(S[6].cpu(), S0[6])


# ------------------------------------------------------------------- decode --

@pytest.mark.parametrize("access", [0, 1, 2])   # auto (here cache-resident), streaming, cache-resident
@pytest.mark.parametrize("normalized", [False, True])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_decode_steps(normalized, dtype, d, access):
    banner("decode normalized=%s dtype=%s d=%d access=%d" % (normalized, dtype, d, access))
    N, H, steps = 3, 4, 12
    S0 = randn((N, H, d, d), 80, 0.01)
    z0 = randn((N, H, d), 81, 0.01).abs() + 1.0 if normalized else None
    S_dev = S0.clone().to(DEV)
    z_dev = None if z0 is None else z0.clone().to(DEV)
    S_ref, z_ref = S0.numpy().astype(np.float64), None if z0 is None else z0.numpy().astype(np.float64)
    shift = 1.0 if normalized else 0.0
    for t in range(steps):
        q, k, v = (randn((N, H, d), 100 * t + i, 1.0, shift if i < 2 else 0.0, dtype=dtype)
                   for i in range(3))
        y = api.la_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), S_dev, z_dev, normalized=normalized,
                               state_access=access)
        yr, S_ref, z_new = O.decode_step(q, k, v, S_ref, z_ref, normalized)
        if normalized:
            z_ref = z_new
        tol = TOL_BF16 if dtype == torch.bfloat16 else TOL_F32
        assert rel_err(np64(y), yr.reshape(N, H * d)) <= tol
    assert rel_err(np64(S_dev), S_ref) <= 1e-5


def test_decode_gated():
    banner("decode gated")
    N, H, d = 4, 8, 128
    S0 = randn((N, H, d, d), 90, 0.01)
    q, k, v = (randn((N, H, d), 91 + i, dtype=torch.bfloat16) for i in range(3))
    x = randn((N, H * d), 94, dtype=torch.bfloat16)
    for odt in (torch.float32, torch.bfloat16):
        S_dev = S0.clone().to(DEV)
        y = api.la_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), S_dev, None, x.to(DEV),
                               out_dtype=odt)
        yr, _, _ = O.decode_step(q, k, v, S0, None, False)
        ref = O.gate(yr.reshape(N, H * d), x, None, 0, 1e-6)
        if odt == torch.float32:
            assert rel_err(np64(y), ref) <= TOL_BF16
        else:
            rms = np.sqrt(np.mean(ref ** 2))
            assert (np.abs(np64(y) - ref) <= 2.0 ** -8 * np.abs(ref) + TOL_BF16 * rms).all()


def test_decode_workload_steps():
    """64 sequences x 64 heads x d=128, fp32 state N(0, 0.01): 10 steps, both modes."""
    w = inputs.WORKLOADS["decode_64x64"]
    for normalized in (False, True):
        banner("decode_64x64 normalized=%s" % normalized)
        S0, z0 = inputs.decode_state(w, device="cpu")
        S_dev, z_dev = S0.to(DEV), z0.to(DEV) if normalized else None
        S_ref, z_ref = S0.numpy().astype(np.float64), z0.numpy().astype(np.float64)
        for step in range(10):
            q, k, v = inputs.decode_token(w, step, device="cpu")
            y = api.la_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), S_dev, z_dev,
                                   normalized=normalized)
            if normalized:
                # the numerator from the same state, for the denominator below
                num, _, _ = O.decode_step(q, k, v, S_ref, None, False)
            yr, S_ref, z_new = O.decode_step(q, k, v, S_ref, z_ref if normalized else None,
                                             normalized)
            got = np64(y)
            if normalized:
                z_ref = z_new
                # the unguarded denominator phi(q).z can pass near zero: compare
                # the rows (token, head) whose oracle |den| = |num / y| >= 0.5
                num = num.reshape(w.N, w.H, w.d)
                yn = yr.reshape(w.N, w.H, w.d)
                j = np.abs(num).argmax(axis=-1)[..., None]
                den = np.take_along_axis(num, j, -1)[..., 0] / np.take_along_axis(yn, j, -1)[..., 0]
                keep = (np.abs(den) >= 0.5).repeat(w.d, axis=1).reshape(w.N, w.H * w.d)
                yr = yr.reshape(w.N, w.H * w.d)
                assert rel_err(got[keep], yr[keep]) <= TOL_BF16
            else:
                assert rel_err(got, yr.reshape(w.N, w.H * w.d)) <= TOL_BF16
        assert rel_err(np64(S_dev), S_ref) <= 1e-5


# ------------------------------------------------------------- invariances --

def test_prefill_equals_decode_and_chaining():
    banner("prefill == decode, chaining")
    T, H, d = 40, 2, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 110 + i, s, dtype=torch.bfloat16).to(DEV) for i in range(3))
    out, S, _ = api.la_prefill(q, k, v)
    # the same tokens one at a time through the decode entry point
    Sd = torch.zeros((1, H, d, d), device=DEV)
    ys = [api.la_decode_step(q[:, t], k[:, t], v[:, t], Sd) for t in range(T)]
    yd = torch.stack(ys, dim=1)
    assert rel_err(np64(yd), np64(out)) <= TOL_BF16
    assert rel_err(np64(Sd), np64(S)) <= 1e-3
    # chunked prefill through state_out -> state_in
    out1, S1, _ = api.la_prefill(q[:, :25], k[:, :25], v[:, :25])
    out2, S2, _ = api.la_prefill(q[:, 25:], k[:, 25:], v[:, 25:], None, None, S1)
    assert rel_err(np64(torch.cat([out1, out2], dim=1)), np64(out)) <= TOL_BF16
    assert rel_err(np64(S2), np64(S)) <= 1e-3


def test_deterministic_and_fully_written():
    banner("determinism")
    T, H, d = 5000, 4, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 120 + i, s, dtype=torch.bfloat16).to(DEV) for i in range(3))
    x = randn((1, T, H * d), 123, dtype=torch.bfloat16).to(DEV)
    a, Sa, _ = api.la_prefill(q, k, v, x, chunk_tokens=1024)
    b, Sb, _ = api.la_prefill(q, k, v, x, chunk_tokens=1024)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(Sa, Sb)
    assert torch.isfinite(a).all() and torch.isfinite(Sa).all()


def test_state_alias_in_place():
    banner("state_out aliasing state_in")
    T, H, d = 300, 2, 128
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((1, T, H, d), 130 + i, s, dtype=torch.bfloat16) for i in range(3))
    S0 = randn((1, H, d, d), 133, 0.05)
    ref, Sref, _ = oracle_forward(q, k, v, None, S0)
    import ctypes

    from linear_attention_long_amd import _lib
    lib = _lib.load()
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    S = S0.clone().to(DEV)
    out = torch.empty((1, T, H * d), device=DEV)
    for chunk in (0, 64):
        S.copy_(S0.to(DEV))
        opt = _lib.options(chunk_tokens=chunk)
        nb = lib.la_prefill_workspace_bytes(1, T, H, d, 1, 0, ctypes.byref(opt))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
        st = lib.la_prefill(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), None, None, S.data_ptr(),
                            None, out.data_ptr(), S.data_ptr(), None, 1, T, H, d, 1, 0,
                            ctypes.byref(opt), ws.data_ptr(), nb, None)
        assert st == 0
        torch.cuda.synchronize()
        assert rel_err(np64(out), ref) <= TOL_BF16
        assert rel_err(np64(S), Sref) <= TOL_BF16


@pytest.mark.parametrize("normalized", [False, True])
def test_decode_access_modes_agree(normalized):
    """Streaming (non-temporal, one workgroup per sequence-head) and
    cache-resident (plain, four workgroups) state access: the state update is
    elementwise and identical, so S (and z) agree bit for bit; y only
    reassociates its sum over rows."""
    banner("decode access modes, normalized=%s" % normalized)
    N, H, d = 5, 6, 128
    S0 = randn((N, H, d, d), 90, 0.01).to(DEV)
    z0 = (randn((N, H, d), 91, 0.01).abs() + 1.0).to(DEV) if normalized else None
    shift = 1.0 if normalized else 0.0
    Ss = {a: S0.clone() for a in (1, 2)}
    zs = {a: None if z0 is None else z0.clone() for a in (1, 2)}
    for t in range(6):
        q, k, v = (randn((N, H, d), 300 * t + i, 1.0, shift if i < 2 else 0.0,
                         dtype=torch.bfloat16).to(DEV) for i in range(3))
        ys = {a: api.la_decode_step(q, k, v, Ss[a], zs[a], normalized=normalized, state_access=a)
              for a in (1, 2)}
        torch.cuda.synchronize()
        assert torch.equal(Ss[1], Ss[2])
        if normalized:
            assert torch.equal(zs[1], zs[2])
        assert rel_err(np64(ys[1]), np64(ys[2])) <= 1e-5
