"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (default block and chunk choice).  The oracle computes the exact fp64
recurrence over every token but emits outputs only at sampled tokens; the
final states are compared in full.

Samples: every token around each chunk boundary and block boundary of the
first chunks, the first and last token of every sequence, and seeded random
tokens; for the 1M-token sequence also every token of the 256-token blocks
0, 1, 2047, 2048 and 4095 and 4096 seeded random tokens.  Metric: max|err| /
rms(ref) over the sampled outputs (1e-2 for bf16 inputs) and over every
final-state element.  The decode workload is compared at every step.
"""
import numpy as np
import pytest
import torch

from linear_attention_long_amd import _lib, api, inputs
from oracle import oracle as O
from tests._util import banner, np64, rel_err

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2


def chunk_tokens(varlen, num_seqs, total, max_len, H, d):
    """Chunk length of the default plan (printed with its kernels) and whether
    the device chooses it (then the returned length is an upper bound)."""
    p = _lib.plan(varlen, num_seqs, total, max_len, H, d, _lib.LA_DTYPE_BF16,
                  _lib.LA_DTYPE_F32, _lib.options(gated=True))
    print("plan: chunk %d%s, %d main workgroups, kernels %s"
          % (p.chunk_tokens, " (bound; chosen on the device)" if p.chunk_on_device else "",
             p.main_workgroups, p.kernel_names()))
    return p.chunk_tokens, bool(p.chunk_on_device)


def sample_tokens(starts, ends, chunk, nrand, seed, every64=False):
    """Sequence ends, tokens around each chunk start (every 64-token boundary
    when the chunk length is chosen on the device), and seeded random ones."""
    idx = set()
    rng = np.random.default_rng(seed)
    for a, b in zip(starts, ends):
        if b <= a:
            continue
        idx.update([a, b - 1])
        if every64:
            for c0 in range(a, b, 64):
                for off in (-1, 0):
                    if a <= c0 + off < b:
                        idx.add(c0 + off)
            continue
        for c0 in range(a, b, chunk):
            for off in (-2, -1, 0, 1, 31, 32, 33, 63, 64):
                t = c0 + off
                if a <= t < b:
                    idx.add(t)
    total = ends[-1]
    idx.update(rng.integers(0, total, size=nrand).tolist())
    return np.array(sorted(idx), dtype=np.int64)


def test_prefill_1m_workload_sampled():
    w = inputs.WORKLOADS["prefill_1m"]
    banner("prefill_1m workload (sampled)")
    q, k, v, x = inputs.prefill_inputs(w, device="cuda")
    out, S, _ = api.la_prefill(q, k, v, x)
    torch.cuda.synchronize()
    C, dev = chunk_tokens(False, 1, w.T, w.T, w.H, w.d)
    idx = sample_tokens([0], [w.T], C, 4096, 7, every64=dev)
    blocks = np.concatenate([np.arange(256 * b, 256 * (b + 1)) for b in (0, 1, 2047, 2048, 4095)])
    idx = np.union1d(idx, blocks).astype(np.int64)
    got = np64(out[0, torch.from_numpy(idx).cuda()])
    S_got = np64(S)
    del out, S
    qc, kc, vc = (t[0].float().cpu() for t in (q, k, v))
    xs = x[0, torch.from_numpy(idx).cuda()].float().cpu()
    del q, k, v, x
    torch.cuda.empty_cache()
    y, S_ref, _ = O.prefill_sampled_f32(qc, kc, vc, idx, nthreads=w.H)
    ref = O.gate(y.reshape(len(idx), w.H * w.d), xs, None, 0, 1e-6)
    e_out, e_S = rel_err(got, ref), rel_err(S_got, S_ref)
    print("prefill_1m: %d sampled tokens, rel err out %.3e state %.3e" % (len(idx), e_out, e_S))
    assert e_out <= TOL_BF16 and e_S <= TOL_BF16


def test_prefill_512k_normalized_half_chunk_state_pass():
    """The normalised mode through the plan of long gated prefills (chunk-state
    pass on half chunks, whose increments carry the column sums of phi(k) for
    z): 524,288 tokens x 8 heads, gated, against the oracle's normalised
    recurrence at sampled tokens, final S and z in full."""
    T, H, d = 1 << 19, 8, 128
    banner("prefill 512K normalized (half-chunk state pass)")
    g = torch.Generator(device="cuda").manual_seed(31)
    s = 1.0 / np.sqrt(d)
    q, k, v = ((torch.randn((1, T, H, d), generator=g, device="cuda") * s).to(torch.bfloat16)
               for _ in range(3))
    x = torch.randn((1, T, H * d), generator=g, device="cuda").to(torch.bfloat16)
    out, S, z = api.la_prefill(q, k, v, x, normalized=True)
    torch.cuda.synchronize()
    C, dev = chunk_tokens(False, 1, T, T, H, d)
    assert C >= 8192 and not dev  # the half-chunk state pass applies
    idx = sample_tokens([0], [T], C, 2048, 9)
    got = np64(out[0, torch.from_numpy(idx).cuda()])
    S_got, z_got = np64(S), np64(z)
    del out, S, z
    qc, kc, vc = (t[0].float().cpu() for t in (q, k, v))
    xs = x[0, torch.from_numpy(idx).cuda()].float().cpu()
    del q, k, v, x
    torch.cuda.empty_cache()
    y, S_ref, z_ref = O.prefill_sampled_f32(qc, kc, vc, idx, normalized=True, nthreads=H)
    ref = O.gate(y.reshape(len(idx), H * d), xs, None, 0, 1e-6)
    e_out, e_S, e_z = rel_err(got, ref), rel_err(S_got, S_ref), rel_err(z_got, z_ref)
    print("prefill 512K normalized: %d sampled tokens, rel err out %.3e state %.3e z %.3e"
          % (len(idx), e_out, e_S, e_z))
    assert e_out <= TOL_BF16 and e_S <= TOL_BF16 and e_z <= TOL_BF16


def test_prefill_4m_past_32bit_offsets():
    """One 4,194,307-token sequence (the pages' 4M-token inference context),
    8 heads of 128, gated: each of q, k, v holds 4.29e9 elements, so the last
    tokens lie past 2^32 elements and the tokens past 2,097,152 past 2^31 --
    any 32-bit offset in a kernel would show.  Sampled as the 1M-token case,
    plus every token of the first and last blocks and tokens around the 2^31
    and 2^32 element marks."""
    w = inputs.WORKLOADS["prefill_1m"]
    T = (1 << 22) + 3
    banner("prefill, T=%d (offsets past 2^32 elements)" % T)
    q, k, v, x = inputs.prefill_inputs(w, T=T, device="cuda")
    out, S, _ = api.la_prefill(q, k, v, x)
    torch.cuda.synchronize()
    C, dev = chunk_tokens(False, 1, T, T, w.H, w.d)
    idx = sample_tokens([0], [T], C, 2048, 17, every64=dev)
    marks = np.concatenate([np.arange(0, 64), np.arange(T - 64, T),
                            np.arange((1 << 21) - 3, (1 << 21) + 3), np.arange((1 << 22) - 3, T)])
    idx = np.union1d(idx, marks).astype(np.int64)
    got = np64(out[0, torch.from_numpy(idx).cuda()])
    S_got = np64(S)
    del out, S
    qc, kc, vc = (t[0].float().cpu() for t in (q, k, v))
    xs = x[0, torch.from_numpy(idx).cuda()].float().cpu()
    del q, k, v, x
    torch.cuda.empty_cache()
    y, S_ref, _ = O.prefill_sampled_f32(qc, kc, vc, idx, nthreads=w.H)
    ref = O.gate(y.reshape(len(idx), w.H * w.d), xs, None, 0, 1e-6)
    e_out, e_S = rel_err(got, ref), rel_err(S_got, S_ref)
    print("prefill T=%d: %d sampled tokens, rel err out %.3e state %.3e" % (T, len(idx), e_out, e_S))
    assert e_out <= TOL_BF16 and e_S <= TOL_BF16


def test_varlen_512k_workload_sampled():
    w = inputs.WORKLOADS["varlen_512k"]
    banner("varlen_512k workload (sampled)")
    q, k, v, x, cu = inputs.varlen_inputs(w, device="cuda")
    lengths = (cu[1:] - cu[:-1]).tolist()
    out, S, _ = api.la_prefill_varlen(q, k, v, cu.cuda(), max(lengths), x)
    torch.cuda.synchronize()
    C, dev = chunk_tokens(True, len(lengths), w.total_T, max(lengths), w.H, w.d)
    idx = sample_tokens(cu[:-1].tolist(), cu[1:].tolist(), C, 512, 11, every64=dev)
    got = np64(out[torch.from_numpy(idx).cuda()])
    S_got = np64(S)
    del out, S
    qc, kc, vc = (t.float().cpu() for t in (q, k, v))
    xs = x[torch.from_numpy(idx).cuda()].float().cpu()
    del q, k, v, x
    torch.cuda.empty_cache()
    y, S_ref, _ = O.prefill_sampled_f32(qc, kc, vc, idx, cu_seqlens=cu.numpy(), nthreads=16)
    ref = O.gate(y.reshape(len(idx), w.H * w.d), xs, None, 0, 1e-6)
    e_out, e_S = rel_err(got, ref), rel_err(S_got, S_ref)
    print("varlen_512k: %d sequences, %d sampled tokens, rel err out %.3e state %.3e"
          % (len(lengths), len(idx), e_out, e_S))
    assert e_out <= TOL_BF16 and e_S <= TOL_BF16


def _decode_outputs(w, normalized):
    """Every step's y [steps, N, H*d] (fp32, on the GPU), the final state and
    normaliser, and the initial ones, for the decode workload."""
    S0, z0 = inputs.decode_state(w, device="cuda")
    S = S0.clone()
    z = z0.clone() if normalized else None
    toks = [inputs.decode_token(w, s, device="cuda") for s in range(w.steps)]
    Y = torch.empty((w.steps, w.N, w.H * w.d), dtype=torch.float32, device="cuda")
    for s in range(w.steps):
        api.la_decode_step(*toks[s], S, z, normalized=normalized, out=Y[s])
    torch.cuda.synchronize()
    return toks, Y, S, z, S0, z0


@pytest.mark.parametrize("normalized", [False, True])
def test_decode_workload_1000_steps(normalized):
    """64 x 64 x d=128 decode, 1000 steps from S0 (and z0) ~ N(0, 0.01): every
    step's output, the final state and normaliser of every (sequence, head),
    against the oracle run as 1000-token prefills from the same state, 16
    sequences at a time.  Normalised mode: the features can be negative, so
    denominators phi(q).z come arbitrarily close to zero; outputs are compared
    on the (token, head) rows whose oracle denominator has magnitude >= 0.5,
    and the excluded count is printed.  The denominator is num / y of the
    oracle's unnormalised and normalised runs (same state, same tokens)."""
    w = inputs.WORKLOADS["decode_64x64"]
    banner("decode_64x64 workload, %d steps, normalized=%s" % (w.steps, normalized))
    toks, Y, S, z, S0, z0 = _decode_outputs(w, normalized)
    got_S = np64(S)
    got_z = np64(z) if normalized else None
    del S, z
    steps, N, H, d = w.steps, w.N, w.H, w.d
    S0c, z0c = S0.cpu(), z0.cpu()
    per = 16
    max_err, sumsq, cnt, excluded = 0.0, 0.0, 0, 0
    S_ref = np.zeros((N, H, d, d))
    z_ref = np.zeros((N, H, d))
    for n0 in range(0, N, per):
        n1 = min(N, n0 + per)
        # sequences n0..n1-1 as 1000-token sequences: [nb * steps, H, d]
        qs, ks, vs = (torch.stack([t[i][n0:n1] for t in toks], dim=1).reshape(-1, H, d)
                      .float().cpu() for i in range(3))
        cu = np.arange(0, (n1 - n0) * steps + 1, steps, dtype=np.int64)
        allidx = np.arange((n1 - n0) * steps, dtype=np.int64)
        yr, Sr, zr = O.prefill_sampled_f32(qs, ks, vs, allidx, cu_seqlens=cu,
                                           state_in=S0c[n0:n1], z_in=z0c[n0:n1] if normalized
                                           else None, normalized=normalized, nthreads=16)
        S_ref[n0:n1] = Sr
        z_ref[n0:n1] = zr
        got = np64(Y[:, n0:n1].permute(1, 0, 2).reshape(-1, H, d))
        if normalized:
            num, _, _ = O.prefill_sampled_f32(qs, ks, vs, allidx, cu_seqlens=cu,
                                              state_in=S0c[n0:n1], nthreads=16)
            j = np.abs(num).argmax(axis=-1)[..., None]
            den = np.take_along_axis(num, j, -1)[..., 0] / np.take_along_axis(yr, j, -1)[..., 0]
            keep = np.abs(den) >= 0.5
            excluded += int((~keep).sum())
            got, yr = got[keep], yr[keep]
        max_err = max(max_err, float(np.abs(got - yr).max()))
        sumsq += float((yr * yr).sum())
        cnt += yr.size
        del qs, ks, vs, yr, got
    e_y = max_err / np.sqrt(sumsq / cnt)
    e_S = rel_err(got_S, S_ref)
    msg = "decode 1000 steps (%s): rel err every step's y %.3e, state %.3e" % (
        "normalized" if normalized else "plain", e_y, e_S)
    if normalized:
        e_z = rel_err(got_z, z_ref)
        msg += ", z %.3e; %d of %d (token, head) rows excluded (|den| < 0.5)" % (
            e_z, excluded, steps * N * H)
        assert e_z <= 1e-5
    print(msg)
    assert e_S <= 1e-4 and e_y <= TOL_BF16
