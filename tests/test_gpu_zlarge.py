"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (default block and chunk choice).  The oracle computes the exact fp64
recurrence over every token but emits outputs only at sampled tokens; the
final states are compared in full.

Samples: every token around each chunk boundary and block boundary of the
first chunks, the first and last token of every sequence, and seeded random
tokens.  Metric: max|err| / rms(ref) over the sampled outputs (1e-2 for bf16
inputs) and over every final-state element.
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
    idx = sample_tokens([0], [w.T], C, 512, 7, every64=dev)
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


def test_decode_workload_1000_steps():
    """64 x 64 x d=128 decode, 1000 steps from S0 ~ N(0, 0.01): the final
    state of every (sequence, head) and the last step's outputs, against the
    oracle run as a 1000-token prefill from the same state."""
    w = inputs.WORKLOADS["decode_64x64"]
    banner("decode_64x64 workload, %d steps" % w.steps)
    S0, _ = inputs.decode_state(w, device="cuda")
    S = S0.clone()
    toks = [inputs.decode_token(w, s, device="cuda") for s in range(w.steps)]
    for s in range(w.steps):
        y = api.la_decode_step(*toks[s], S)
    torch.cuda.synchronize()
    got_S, got_y = np64(S), np64(y)
    # packed as 64 sequences of 1000 tokens: [N * steps, H, d]
    qs, ks, vs = (torch.stack([t[i] for t in toks], dim=1).reshape(w.N * w.steps, w.H, w.d)
                  .float().cpu() for i in range(3))
    cu = np.arange(0, w.N * w.steps + 1, w.steps, dtype=np.int64)
    last = cu[1:] - 1
    yr, S_ref, _ = O.prefill_sampled_f32(qs, ks, vs, last, cu_seqlens=cu, state_in=S0.cpu(),
                                         nthreads=16)
    e_S = rel_err(got_S, S_ref)
    e_y = rel_err(got_y, yr.reshape(w.N, w.H * w.d))
    print("decode 1000 steps: rel err state %.3e last y %.3e" % (e_S, e_y))
    assert e_S <= 1e-4 and e_y <= TOL_BF16
