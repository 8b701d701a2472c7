"""The calls under HIP graph capture (torch.cuda.graph): decode (both state
access forms), the fused and chunked prefill (cooperative launch), a packed
prefill with state slots, a serving step, the softmax attention layer and a
whole layer (both projections around the path) are captured once and
replayed several times, with eager work
and synchronisation between replays; every replay must reproduce the eager
result bit for bit.  (No call records a memset node: buffers that must start
at zero are cleared by kernels.)"""
import pytest
import torch

from linear_attention_long_amd import api, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def rnd(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(dtype)


def capture(fn):
    """Warm fn on a side stream, then capture it; returns (graph, outputs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    return g, outs


def replay_and_check(g, reset, outs, refs, n=4):
    for r in range(n):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), "replay %d differs" % r
        # eager work between replays
        assert torch.isfinite(outs[0].float().sum() * 0.5).item()


@pytest.mark.parametrize("access", [0, 1])
def test_graph_decode(access):
    """Both state access forms: the default for this small state
    (cache-resident) and the streaming form."""
    N, H, d = 8, 8, 128
    q, k, v = rnd((N, H, d), 1), rnd((N, H, d), 2), rnd((N, H, d), 3)
    S0 = rnd((N, H, d, d), 4, 0.01, torch.float32)
    S_e = S0.clone()
    y_e = api.la_decode_step(q, k, v, S_e, state_access=access)
    S_g = S0.clone()
    g, (y_g,) = capture(lambda: (api.la_decode_step(q, k, v, S_g, state_access=access),))
    replay_and_check(g, lambda: S_g.copy_(S0), [y_g, S_g], [y_e, S_e])


@pytest.mark.parametrize("T", [4096, 32768])
def test_graph_prefill_fused_chunked(T):
    H, d = 8, 128
    q, k, v = (rnd((1, T, H, d), 10 + i, 128 ** -0.5) for i in range(3))
    x = rnd((1, T, H * d), 13)
    out_e, S_e, _ = api.la_prefill(q, k, v, x)
    g, (out_g, S_g) = capture(lambda: api.la_prefill(q, k, v, x)[:2])
    replay_and_check(g, lambda: out_g.zero_(), [out_g, S_g], [out_e, S_e])


def test_graph_varlen_with_slots_and_serving_step():
    H, d = 8, 128
    lengths = [700, 1, 0, 2000, 64]
    cu = inputs.cu_from_lengths(lengths).to(DEV)
    total = int(cu[-1])
    q, k, v = (rnd((total, H, d), 20 + i, 128 ** -0.5) for i in range(3))
    x = rnd((total, H * d), 23)
    pool0 = rnd((9, H, d, d), 24, 0.02, torch.float32)
    slots = torch.tensor([4, 0, 7, 2, 8], dtype=torch.int32, device=DEV)
    pool_e = pool0.clone()
    out_e, _, _ = api.la_prefill_varlen(q, k, v, cu, max(lengths), x, None, pool_e,
                                        state_slots=slots)
    pool_g = pool0.clone()
    g, (out_g,) = capture(lambda: (api.la_prefill_varlen(q, k, v, cu, max(lengths), x, None,
                                                         pool_g, state_slots=slots)[0],))
    replay_and_check(g, lambda: pool_g.copy_(pool0), [out_g, pool_g], [out_e, pool_e])

    # a serving step: 3 decode tokens (rows 0..2), then chunks of 500 and 37 tokens
    nd = 3
    rows = nd + 537
    dslots = torch.tensor([1, 3, 5], dtype=torch.int32, device=DEV)
    pslots = torch.tensor([6, 0], dtype=torch.int32, device=DEV)
    pcu = torch.tensor([0, 500, 537], dtype=torch.int32, device=DEV)
    qs, ks, vs, xs = q[:rows], k[:rows], v[:rows], x[:rows]
    cur = torch.cuda.current_stream()
    pool_e = pool0.clone()
    out_e = api.la_serve_step(qs, ks, vs, pool_e, dslots, pcu, pslots, 500, x=xs,
                              decode_stream=cur, prefill_stream=cur)
    pool_g = pool0.clone()

    def step():
        s = torch.cuda.current_stream()
        return (api.la_serve_step(qs, ks, vs, pool_g, dslots, pcu, pslots, 500, x=xs,
                                  decode_stream=s, prefill_stream=s),)

    g, (out_g,) = capture(step)
    replay_and_check(g, lambda: pool_g.copy_(pool0), [out_g, pool_g], [out_e, pool_e])


@pytest.mark.parametrize("precision", [0, 1, 2])
def test_graph_softmax_packed(precision):
    # the softmax layer on a packed batch: ordering pass (atomics), rotation and
    # attention kernels captured together
    lengths = [700, 1, 300, 2048]
    T, H, Hkv, d = sum(lengths), 8, 2, 128
    q, k, v = rnd((T, H, d), 11), rnd((T, Hkv, d), 12), rnd((T, Hkv, d), 13)
    cu = torch.tensor([0, 700, 701, 1001, T], dtype=torch.int32, device=DEV)
    kw = dict(rope_base=1e7, out_dtype=torch.float32, return_lse=True, precision=precision)
    o_e, l_e = api.la_softmax_attention_varlen(q, k, v, cu, 2048, **kw)
    g, (o_g, l_g) = capture(lambda: api.la_softmax_attention_varlen(q, k, v, cu, 2048, **kw))
    replay_and_check(g, lambda: (o_g.zero_(), l_g.zero_()), [o_g, l_g], [o_e, l_e])


def test_graph_whole_layer():
    """Input projection, the path (features given, gated, bf16 out) and the
    output projection captured as one graph."""
    T, K, H, d, N = 2048, 1024, 8, 128, 2048
    F = H * d
    h = rnd((T, K), 11)
    w = rnd((4 * F, K), 12, K ** -0.5)
    wo = rnd((N, F), 13, F ** -0.5)

    def layer():
        q, k, v, xg = api.la_qkvx_projection(h, w, F)
        y = api.la_prefill(q.view(T, H, d), k.view(T, H, d), v.view(T, H, d), xg,
                           featurized=True, out_dtype=torch.bfloat16, return_state=False)[0]
        return (api.la_out_projection(y.view(T, F), wo, out_dtype=torch.float32),)

    (z_e,) = layer()
    torch.cuda.synchronize()
    g, (z_g,) = capture(layer)
    replay_and_check(g, lambda: z_g.zero_(), [z_g], [z_e])
