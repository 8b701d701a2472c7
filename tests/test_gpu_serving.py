"""GPU parity of the serving calls: state slots (per-request rows of a state
pool, updated in place) for decode and packed prefill, and whole request
streams driven through la_schedule_step + la_serve_step (chunked prefill and
decode on two streams), against the oracle run over each request's tokens."""
import numpy as np
import pytest
import torch

from linear_attention_long_amd import api, inputs, serving
from oracle import oracle as O
from tests._util import banner, np64, randn, rel_err

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
DEV = "cuda"


@pytest.mark.parametrize("normalized", [False, True])
def test_decode_with_state_slots(normalized):
    banner("decode with state slots normalized=%s" % normalized)
    rows, H, d = 10, 4, 128
    slots = [7, 2, 9, 0]
    N = len(slots)
    pool0 = randn((rows, H, d, d), 200, 0.01)
    zp0 = randn((rows, H, d), 201, 0.01).abs() + 1.0 if normalized else None
    q, k, v = (randn((N, H, d), 202 + i, dtype=torch.bfloat16) for i in range(3))
    pool = pool0.to(DEV)
    zp = zp0.to(DEV) if normalized else None
    y = api.la_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), pool, zp, normalized=normalized,
                           state_slots=torch.tensor(slots, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    for n, r in enumerate(slots):
        yr, Sr, zr = O.forward(q[n:n + 1], k[n:n + 1], v[n:n + 1], state_in=pool0[r:r + 1],
                               z_in=None if zp0 is None else zp0[r:r + 1], normalized=normalized)
        assert rel_err(np64(y[n]).reshape(-1), yr.reshape(-1)) <= TOL_BF16
        assert rel_err(np64(pool[r]), Sr[0]) <= 1e-4
        if normalized:
            assert rel_err(np64(zp[r]), zr[0]) <= 1e-5
    for r in set(range(rows)) - set(slots):   # rows no sequence names stay as they were
        assert torch.equal(pool[r].cpu(), pool0[r])


@pytest.mark.parametrize("chunk", [0, 512])
def test_varlen_with_state_slots_in_place(chunk):
    banner("varlen with state slots in place, chunk=%d" % chunk)
    lengths = [300, 1, 0, 2500, 64]
    slots = [5, 11, 3, 0, 8]
    rows, H, d = 12, 8, 128
    cu = inputs.cu_from_lengths(lengths)
    total = int(cu[-1])
    s = 1.0 / np.sqrt(d)
    q, k, v = (randn((total, H, d), 210 + i, s, dtype=torch.bfloat16) for i in range(3))
    x = randn((total, H * d), 213, dtype=torch.bfloat16)
    pool0 = randn((rows, H, d, d), 214, 0.05)
    pool = pool0.to(DEV)
    out, S, _ = api.la_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lengths),
                                      x.to(DEV), None, pool, state_slots=torch.tensor(
                                          slots, dtype=torch.int32, device=DEV),
                                      chunk_tokens=chunk)
    torch.cuda.synchronize()
    assert S is pool
    ref, Sref, _ = O.forward(q, k, v, x, None, cu_seqlens=cu.numpy(),
                             state_in=pool0[torch.tensor(slots)], gated=True)
    assert rel_err(np64(out), ref) <= TOL_BF16
    got = np64(pool[torch.tensor(slots, device=DEV)])
    assert rel_err(got, Sref) <= TOL_BF16
    assert torch.equal(pool[3].cpu(), pool0[3])           # the empty sequence keeps its state
    for r in set(range(rows)) - set(slots):
        assert torch.equal(pool[r].cpu(), pool0[r])


@pytest.mark.parametrize("gated,normalized,budget,two", [(True, False, 2048, True),
                                                         (False, True, 1500, True),
                                                         (True, False, 1024, False)])
def test_serving_streams_match_oracle(gated, normalized, budget, two):
    """Five requests (prompts 3000, 1, 37, 5000, 700; then 6 decoded tokens
    each) under a small token budget: prompts are split across steps and
    decode tokens share steps with prefill chunks (on two streams, or one)."""
    banner("serving gated=%s normalized=%s budget=%d two_streams=%s"
           % (gated, normalized, budget, two))
    H, d = 4, 128
    prompts = [3000, 1, 37, 5000, 700]
    ndec = 6
    s = 1.0 / np.sqrt(d)
    reqs, host = [], []
    for i, p in enumerate(prompts):
        T = p + ndec
        if normalized:
            qh, kh = (randn((T, H, d), 300 + 10 * i + j, 0.5, 1.0, dtype=torch.bfloat16) for j in range(2))
        else:
            qh, kh = (randn((T, H, d), 300 + 10 * i + j, s, dtype=torch.bfloat16) for j in range(2))
        vh = randn((T, H, d), 302 + 10 * i, dtype=torch.bfloat16)
        xh = randn((T, H * d), 303 + 10 * i, dtype=torch.bfloat16) if gated else None
        host.append((qh, kh, vh, xh))
        reqs.append(serving.Request(q=qh.to(DEV), k=kh.to(DEV), v=vh.to(DEV), prompt=p,
                                    x=None if xh is None else xh.to(DEV), slot=2 * i + 1))
    rows = 2 * len(prompts) + 1
    pool0 = randn((rows, H, d, d), 350, 0.02)
    zp0 = torch.ones((rows, H, d)) if normalized else None
    pool = pool0.to(DEV)
    zp = zp0.to(DEV) if normalized else None
    steps = []
    nsteps = serving.run(reqs, pool, z_pool=zp, normalized=normalized, max_batched_tokens=budget,
                         two_streams=two, on_step=lambda i, st: steps.append((st.num_decode, st.num_prefill,
                                                             st.prefill_tokens)))
    torch.cuda.synchronize()
    # the budget forces mixed steps: some with both decoders and chunks
    assert any(a > 0 and b > 0 for a, b, _ in steps), steps
    assert all(a + c <= budget for a, _, c in steps)
    print("serving: %d steps: %s" % (nsteps, steps))
    for i, (r, (qh, kh, vh, xh)) in enumerate(zip(reqs, host)):
        got = np64(torch.cat(r.out))
        ref, Sref, zref = O.forward(qh, kh, vh, xh, None, state_in=pool0[r.slot:r.slot + 1],
                                    z_in=None if zp0 is None else zp0[r.slot:r.slot + 1],
                                    normalized=normalized, gated=gated)
        assert rel_err(got, ref) <= TOL_BF16, i
        assert rel_err(np64(pool[r.slot]), Sref[0]) <= TOL_BF16, i
        if normalized:
            assert rel_err(np64(zp[r.slot]), zref[0]) <= 1e-4, i
    for r in range(0, rows, 2):                     # rows of no request
        assert torch.equal(pool[r].cpu(), pool0[r])
