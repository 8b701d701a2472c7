"""Host-side serving logic: the step scheduler (la_schedule_step) against a
plain Python statement of its policy, and argument checks of the serving and
slot options that reject calls before any HIP call (no GPU needed)."""
import ctypes
import os

import numpy as np
import pytest

from linear_attention_long_amd import _lib, api

INVALID = _lib.LA_ERR_INVALID_ARGUMENT
F32, BF16 = _lib.LA_DTYPE_F32, _lib.LA_DTYPE_BF16
A = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(16)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from linear_attention_long_amd import build

        build.build()
    return _lib.load()


def policy(remaining, budget):
    """The documented policy: decoders first, then prompt chunks in request
    order while the budget lasts."""
    order = [i for i, r in enumerate(remaining) if r == 0]
    chunk = [1] * len(order)
    left = budget - len(order)
    for i, r in enumerate(remaining):
        if r == 0:
            continue
        if left <= 0:
            break
        c = min(r, left)
        order.append(i)
        chunk.append(c)
        left -= c
    return order, chunk


def test_schedule_step_matches_policy(lib):
    rng = np.random.default_rng(5)
    for trial in range(200):
        R = int(rng.integers(0, 12))
        rem = [int(x) if rng.random() < 0.6 else 0 for x in rng.integers(1, 50000, size=R)]
        nd = sum(1 for r in rem if r == 0)
        budget = int(rng.integers(nd, 70000))
        order, chunk, st = api.la_schedule_step(rem, budget)
        eo, ec = policy(rem, budget)
        assert (order, chunk) == (eo, ec), (rem, budget)
        assert st.num_decode == nd and st.num_decode + st.num_prefill == len(order)
        assert st.prefill_tokens == sum(chunk[nd:]) and sum(chunk) <= budget
        assert st.max_chunk == max(chunk[nd:], default=0)


def test_schedule_step_rejects(lib):
    step = _lib.Step()
    o = (ctypes.c_int32 * 4)()
    c = (ctypes.c_int32 * 4)()
    reqs = (_lib.Request * 2)()
    reqs[0].remaining, reqs[1].remaining = 0, -1
    assert lib.la_schedule_step(reqs, 2, 100, o, c, ctypes.byref(step)) == INVALID  # negative
    reqs[1].remaining = 0
    assert lib.la_schedule_step(reqs, 2, 1, o, c, ctypes.byref(step)) == INVALID  # budget < decoders
    assert lib.la_schedule_step(None, 2, 100, o, c, ctypes.byref(step)) == INVALID
    assert lib.la_schedule_step(reqs, -1, 100, o, c, ctypes.byref(step)) == INVALID
    assert lib.la_schedule_step(reqs, 2, 100, o, c, None) == INVALID
    assert lib.la_schedule_step(None, 0, 0, None, None, ctypes.byref(step)) == _lib.LA_OK
    assert (step.num_decode, step.num_prefill, step.prefill_tokens) == (0, 0, 0)


def serve(lib, **kw):
    a = dict(q=A[0], k=A[1], v=A[2], x=None, w=None, pool=A[3], zp=None, rows=8, dslots=A[4],
             nd=2, cu=A[5], pslots=A[6], np_=1, ptok=100, maxc=100, out=A[7], H=2, d=64,
             idt=F32, odt=F32, o=None, ws=None, wsb=0)
    a.update(kw)
    o = a["o"] or _lib.options()
    return lib.la_serve_step(a["q"], a["k"], a["v"], a["x"], a["w"], a["pool"], a["zp"], a["rows"],
                             a["dslots"], a["nd"], a["cu"], a["pslots"], a["np_"], a["ptok"],
                             a["maxc"], a["out"], a["H"], a["d"], a["idt"], a["odt"],
                             ctypes.byref(o), a["ws"], a["wsb"], None, None)


def test_serve_step_rejects(lib):
    assert serve(lib, rows=0) == INVALID
    assert serve(lib, pool=None) == INVALID
    assert serve(lib, dslots=None) == INVALID
    assert serve(lib, pslots=None) == INVALID
    assert serve(lib, cu=None) == INVALID
    assert serve(lib, maxc=101) == INVALID        # longer than the chunks' tokens
    assert serve(lib, np_=0, ptok=5) == INVALID   # tokens without sequences
    assert serve(lib, nd=-1) == INVALID
    assert serve(lib, d=96) == _lib.LA_ERR_UNSUPPORTED
    o = _lib.options()
    o.state_slots = A[8].value
    o.state_rows = 4
    assert serve(lib, o=o) == INVALID             # slots come as arguments here
    # a normalised step needs the z pool (the decode part rejects before any launch)
    assert serve(lib, o=_lib.options(normalized=True)) == INVALID
    assert lib.la_serve_step_workspace_bytes(-1, 0, 0, 1, 2, 64, F32, F32, None) == ctypes.c_size_t(-1).value


def test_slot_option_checks(lib):
    o = _lib.options()
    o.state_slots = A[8].value
    o.state_rows = 0                               # slots need rows >= 1
    assert lib.la_decode_step(A[0], A[1], A[2], None, None, A[3], None, A[4], 2, 2, 64, F32, F32,
                              ctypes.byref(o), None, 0, None) == INVALID
    o.state_rows = 4
    o.state_slots = A[8].value + 2                 # misaligned slot table
    assert lib.la_decode_step(A[0], A[1], A[2], None, None, A[3], None, A[4], 2, 2, 64, F32, F32,
                              ctypes.byref(o), None, 0, None) == INVALID
