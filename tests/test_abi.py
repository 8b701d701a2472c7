"""C-ABI checks that need no GPU: the library loads, exports every function
include/la.h, include/la_softmax.h and include/la_proj.h declare, and rejects invalid calls on
the host.

Every call below fails host validation, so none of them reaches a HIP call;
the fake device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest
import torch

from linear_attention_long_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in ("la.h", "la_softmax.h", "la_proj.h")]

F32, BF16 = _lib.LA_DTYPE_F32, _lib.LA_DTYPE_BF16
INVALID, UNSUPPORTED, WS_SMALL = (_lib.LA_ERR_INVALID_ARGUMENT, _lib.LA_ERR_UNSUPPORTED,
                                  _lib.LA_ERR_WORKSPACE_TOO_SMALL)
SIZE_MAX = ctypes.c_size_t(-1).value

# fake, 256-byte aligned, never dereferenced "device" addresses
A = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(12)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from linear_attention_long_amd import build

        build.build()
    return _lib.load()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+[\s\*]+(la_[a-z_]+)\s*\(", text, re.M)))


def test_header_declares_the_python_export_list():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_default_options(lib):
    o = lib.la_default_options()
    assert (o.block_size, o.normalized, o.gated, o.norm_group, o.chunk_tokens) == (0, 0, 0, 0, 0)
    assert abs(o.rms_eps - 1e-6) < 1e-12
    assert o.featurized == 0 and o.wait_spin_limit == 0 and o.state_access == 0


def test_featurized_inputs_supported_set(lib):
    """Inputs given as features: every prefill configuration but the bf16
    d = 128 matrix-core pass with 64-token blocks, which is refused on the host
    before any device work."""
    bad = ctypes.c_size_t(-1).value
    bf, f32 = _lib.LA_DTYPE_BF16, _lib.LA_DTYPE_F32
    ok = _lib.options(featurized=True)
    assert lib.la_prefill_workspace_bytes(1, 4096, 8, 128, bf, f32, ctypes.byref(ok)) != bad
    assert lib.la_prefill_workspace_bytes(1, 4096, 8, 128, f32, f32, ctypes.byref(ok)) != bad
    assert lib.la_prefill_workspace_bytes(1, 4096, 8, 64, bf, f32, ctypes.byref(ok)) != bad
    b64 = _lib.options(featurized=True, block_size=64)
    assert lib.la_prefill_workspace_bytes(1, 4096, 8, 128, bf, f32, ctypes.byref(b64)) == bad
    odd = _lib.options()
    odd.featurized = 2
    assert lib.la_prefill_workspace_bytes(1, 4096, 8, 128, bf, f32, ctypes.byref(odd)) == bad
    r = _lib.Plan()
    assert lib.la_prefill_plan(0, 1, 4096, 4096, 8, 128, bf, f32, 1, ctypes.byref(b64),
                               ctypes.byref(r)) == _lib.LA_ERR_UNSUPPORTED


def test_status_strings(lib):
    for s in range(6):
        assert lib.la_status_string(s) and lib.la_status_string(s) != b"unknown status"
    assert lib.la_status_string(99) == b"unknown status"


def opt(**kw):
    o = _lib.options()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def test_workspace_queries(lib):
    o = opt()
    # one chunk per sequence, ungated: nothing needed
    assert lib.la_prefill_workspace_bytes(1, 512, 2, 64, F32, F32, ctypes.byref(o)) == 0
    # two 512-token chunks x 2 heads x d^2 floats
    assert lib.la_prefill_workspace_bytes(1, 1024, 2, 64, F32, F32, ctypes.byref(o)) == 2 * 2 * 64 * 64 * 4
    # 1M tokens x 8 heads, ungated: chunk 4096 -> 256 chunks x 8 heads x d^2 floats
    p = _lib.plan(0, 1, 1 << 20, 1 << 20, 8, 128, BF16, F32, o)
    assert (p.chunk_tokens, p.block_size, p.fused_gate) == (4096, 32, 0)
    nb = lib.la_prefill_workspace_bytes(1, 1 << 20, 8, 128, BF16, F32, ctypes.byref(o))
    assert nb == 256 * 8 * 128 * 128 * 4
    g = opt(gated=1)
    nb2 = lib.la_prefill_workspace_bytes(1, 1 << 20, 8, 128, BF16, BF16, ctypes.byref(g))
    pg = _lib.plan(0, 1, 1 << 20, 1 << 20, 8, 128, BF16, BF16, g)
    if pg.fused_gate:
        # fused gate (a device that holds every workgroup): chunk states plus
        # the exchange buffer (4 slots x H x 32 tokens of 8 bytes per chunk)
        # after the call's 256-byte status word
        n = (1 << 20) // pg.chunk_tokens
        assert nb2 == n * 8 * 128 * 128 * 4 + 256 + n * 4 * 8 * 32 * 8
        assert pg.status_offset == n * 8 * 128 * 128 * 4
    else:
        # separate gate with a bf16 output: an fp32 Y buffer
        assert nb2 == nb + (1 << 20) * 8 * 128 * 4
    assert lib.la_decode_workspace_bytes(64, 64, 128, F32, ctypes.byref(g)) == 0
    assert lib.la_decode_workspace_bytes(64, 64, 128, BF16, ctypes.byref(g)) == 64 * 64 * 128 * 4
    # rejected arguments report SIZE_MAX
    assert lib.la_prefill_workspace_bytes(1, 16, 2, 96, F32, F32, ctypes.byref(o)) == SIZE_MAX
    assert lib.la_prefill_workspace_bytes(0, 16, 2, 64, F32, F32, ctypes.byref(o)) == SIZE_MAX
    assert lib.la_prefill_varlen_workspace_bytes(10, 2, 11, 2, 64, F32, F32, ctypes.byref(o)) == SIZE_MAX


def test_prefill_plan(lib):
    o = opt()
    names = lambda *a, **kw: _lib.plan(*a, **kw).kernel_names()
    assert names(0, 1, 512, 512, 2, 64, F32, F32, o) == ["main"]
    assert names(0, 1, 1024, 1024, 2, 64, F32, F32, o) == ["chunk_state", "chunk_scan", "main"]
    assert names(0, 1, 0, 0, 2, 64, F32, F32, o) == ["state_copy"]
    assert names(0, 1, 0, 0, 2, 64, F32, F32, o, has_state_out=False) == []
    assert names(1, 3, 900, 400, 2, 64, F32, F32, o) == ["chunk_table", "state_copy", "main"]
    assert names(1, 3, 1500, 1000, 2, 64, F32, F32, o) == [
        "chunk_table", "chunk_state", "chunk_scan", "main"]
    # fp32 inputs never fuse the gate
    assert names(0, 1, 512, 512, 2, 64, F32, F32, opt(gated=1)) == ["main", "gate"]
    # per-head norm groups or more than 8 heads keep the gate separate
    for g in (opt(gated=1, norm_group=128), opt(gated=1)):
        H = 4 if g.norm_group else 9
        p = _lib.plan(0, 1, 4096, 4096, H, 128, BF16, F32, g)
        assert p.fused_gate == 0 and p.kernel_names()[-2:] == ["main", "gate"]
    p = _lib.plan(0, 2, 2000, 1000, 2, 128, BF16, F32, opt(block_size=64))
    assert p.block_size == 64 and p.main_workgroups == 2 * 2 * 2  # 2 chunks x 2 seqs x H
    p = _lib.plan(0, 2, 2000, 1000, 2, 64, F32, F32, o)
    assert p.block_size == 64
    r = _lib.Plan()
    assert lib.la_prefill_plan(0, 2, 2001, 1000, 2, 64, F32, F32, 1, ctypes.byref(o),
                               ctypes.byref(r)) == INVALID  # total != Bt * T
    assert lib.la_prefill_plan(1, 2, 100, 101, 2, 64, F32, F32, 1, ctypes.byref(o),
                               ctypes.byref(r)) == INVALID  # max_seqlen > total
    assert lib.la_prefill_plan(0, 1, 64, 64, 2, 96, F32, F32, 1, ctypes.byref(o),
                               ctypes.byref(r)) == UNSUPPORTED
    assert lib.la_prefill_plan(0, 1, 64, 64, 2, 64, F32, F32, 1, ctypes.byref(o), None) == INVALID


def test_wait_options_and_status_query(lib):
    """wait_spin_limit takes -1, 0 (default) or a positive bound; the status
    query of a plan without a bounded wait returns at once, and a status word
    with no workspace is an invalid argument (neither touches the device)."""
    for lim in (-1, 0, 1, 1 << 20):
        assert lib.la_prefill_workspace_bytes(1, 4096, 8, 128, BF16, F32,
                                              ctypes.byref(opt(gated=1, wait_spin_limit=lim))) != SIZE_MAX
    assert lib.la_prefill_workspace_bytes(1, 4096, 8, 128, BF16, F32,
                                          ctypes.byref(opt(gated=1, wait_spin_limit=-2))) == SIZE_MAX
    assert prefill(lib, o=opt(wait_spin_limit=-5)) == INVALID
    p = _lib.plan(0, 1, 4096, 4096, 8, 128, BF16, F32, opt())   # ungated: no wait
    assert p.status_offset == -1
    assert lib.la_prefill_wait_status(None, -1, None) == _lib.LA_OK
    assert lib.la_prefill_wait_status(None, 0, None) == INVALID


def prefill(lib, q=A[0], k=A[1], v=A[2], x=None, w=None, si=None, zi=None, out=A[3], so=None,
            zo=None, Bt=1, T=64, H=2, d=64, idt=F32, odt=F32, o=None, ws=None, wsb=0):
    o = o or opt()
    return lib.la_prefill(q, k, v, x, w, si, zi, out, so, zo, Bt, T, H, d, idt, odt,
                          ctypes.byref(o), ws, wsb, None)


def test_prefill_rejects_bad_arguments(lib):
    assert prefill(lib, q=None) == INVALID
    assert prefill(lib, out=None) == INVALID
    assert prefill(lib, q=ctypes.c_void_p(0x10000004)) == INVALID          # misaligned
    assert prefill(lib, d=96) == UNSUPPORTED
    assert prefill(lib, d=0) == INVALID
    assert prefill(lib, H=0) == INVALID
    assert prefill(lib, T=-1) == INVALID
    assert prefill(lib, Bt=0) == INVALID
    assert prefill(lib, idt=7) == INVALID
    assert prefill(lib, Bt=1 << 16, T=1 << 15) == INVALID                # Bt*T past int32 tokens
    assert prefill(lib, H=1 << 15) == UNSUPPORTED                        # H*d past 2^20 features
    assert prefill(lib, o=opt(block_size=48)) == UNSUPPORTED
    assert prefill(lib, o=opt(normalized=2)) == INVALID
    assert prefill(lib, o=opt(gated=1)) == INVALID                         # no gate input
    assert prefill(lib, o=opt(norm_group=100)) == INVALID
    assert prefill(lib, o=opt(rms_eps=-1.0)) == INVALID
    assert prefill(lib, o=opt(chunk_tokens=100)) == INVALID
    assert prefill(lib, zi=A[5]) == INVALID                               # z without normalised mode
    # out overlapping an input
    assert prefill(lib, out=A[0]) == INVALID
    # state_out partly overlapping state_in
    assert prefill(lib, si=A[6], so=ctypes.c_void_p(A[6].value + 256)) == INVALID
    # chunked plan needs a workspace
    o = opt(chunk_tokens=64)
    assert prefill(lib, T=4096, o=o) == INVALID                          # NULL workspace
    need = lib.la_prefill_workspace_bytes(1, 4096, 2, 64, F32, F32, ctypes.byref(o))
    assert need > 0
    assert prefill(lib, T=4096, o=o, ws=A[8], wsb=need - 1) == WS_SMALL


def test_varlen_rejects_bad_arguments(lib):
    o = opt()

    def call(cu=A[9], nseq=2, total=100, maxlen=60, **kw):
        return lib.la_prefill_varlen(A[0], A[1], A[2], None, None, cu, nseq, total, maxlen,
                                     None, None, A[3], None, None, kw.get("H", 2), kw.get("d", 64),
                                     F32, F32, ctypes.byref(kw.get("o", o)), None, 0, None)

    assert call(cu=None) == INVALID
    assert call(nseq=0) == INVALID
    assert call(total=-1) == INVALID
    assert call(maxlen=101) == INVALID
    assert call(d=32) == UNSUPPORTED
    # varlen always needs the chunk table in the workspace
    assert call() == INVALID


def test_decode_rejects_bad_arguments(lib):
    def call(q=A[0], state=A[4], z=None, out=A[3], x=None, N=4, H=2, d=64, o=None, ws=None, wsb=0,
             odt=F32):
        o = o or opt()
        return lib.la_decode_step(q, A[1], A[2], x, None, state, z, out, N, H, d, F32, odt,
                                  ctypes.byref(o), ws, wsb, None)

    assert call(q=None) == INVALID
    assert call(state=None) == INVALID
    assert call(N=-1) == INVALID
    assert call(d=256) == UNSUPPORTED
    assert call(o=opt(normalized=1)) == INVALID          # normalised mode needs z
    assert call(z=A[5]) == INVALID                       # z without normalised mode
    assert call(o=opt(gated=1)) == INVALID               # gate input missing
    assert call(out=A[4]) == INVALID                     # out overlaps the state
    g = opt(gated=1)
    assert call(o=g, x=A[6], odt=BF16) == INVALID        # bf16 gated output needs workspace
    assert call(o=g, x=A[6], odt=BF16, ws=A[7], wsb=16) == WS_SMALL


def test_softmax_default_options(lib):
    o = lib.la_softmax_default_options()
    assert (o.rotary_dim, o.rope_base, o.scale, o.n_timing) == (-1, 10000.0, 0.0, 0)
    assert o.precision == 1  # split operands: within 1e-2 of the output's rms for any bf16 input


def test_softmax_workspace_bytes(lib):
    o = _lib.softmax_options(precision=0)
    # one sequence: rotated q and k only (bf16), each rounded up to 256 bytes
    assert lib.la_softmax_workspace_bytes(1, 1000, 1000, 4, 2, 128, BF16, F32,
                                          ctypes.byref(o)) == 1000 * 4 * 256 + 1000 * 2 * 256
    # packed: plus the count, the order table and the plan's arrays
    nb = lib.la_softmax_workspace_bytes(3, 1000, 600, 4, 4, 128, BF16, BF16, ctypes.byref(o))
    assert nb > 2 * 1000 * 4 * 256
    assert lib.la_softmax_workspace_bytes(1, 0, 0, 4, 4, 128, BF16, F32, ctypes.byref(o)) == 0
    # rejected arguments report SIZE_MAX
    assert lib.la_softmax_workspace_bytes(1, 16, 16, 4, 3, 128, BF16, F32, ctypes.byref(o)) == SIZE_MAX
    assert lib.la_softmax_workspace_bytes(1, 16, 16, 4, 4, 64, BF16, F32, ctypes.byref(o)) == SIZE_MAX
    assert lib.la_softmax_workspace_bytes(1, 16, 17, 4, 4, 128, BF16, F32, ctypes.byref(o)) == SIZE_MAX
    # the split mode adds the bf16 remainders of the rotated q and k
    osp = _lib.softmax_options(precision=1)
    assert lib.la_softmax_workspace_bytes(1, 1000, 1000, 4, 2, 128, BF16, F32,
                                          ctypes.byref(osp)) == 2 * (1000 * 4 * 256 + 1000 * 2 * 256)
    # fp16 operands: the rotated q and k in fp16, no remainders, and v in fp16
    o16 = _lib.softmax_options(precision=2)
    assert lib.la_softmax_workspace_bytes(1, 1000, 1000, 4, 2, 128, BF16, F32,
                                          ctypes.byref(o16)) == 1000 * 4 * 256 + 2 * (1000 * 2 * 256)
    # packed: the work order follows the fp16 v, so mode 2 needs exactly the v
    # bytes more than the single mode for the same batch
    n0 = lib.la_softmax_workspace_bytes(3, 1000, 600, 4, 2, 128, BF16, BF16, ctypes.byref(o))
    n2 = lib.la_softmax_workspace_bytes(3, 1000, 600, 4, 2, 128, BF16, BF16, ctypes.byref(o16))
    assert n2 == n0 + 1000 * 2 * 256
    # the base is not used (nor checked) without rotation
    o0 = _lib.softmax_options(rotary_dim=0, rope_base=0.0)
    assert lib.la_softmax_workspace_bytes(1, 16, 16, 4, 4, 128, BF16, F32, ctypes.byref(o0)) > 0
    o1 = _lib.softmax_options(rope_base=0.0)
    assert lib.la_softmax_workspace_bytes(1, 16, 16, 4, 4, 128, BF16, F32, ctypes.byref(o1)) == SIZE_MAX


def test_softmax_rejects_bad_arguments(lib):
    def call(q=A[0], k=A[1], v=A[2], cu=A[9], nseq=2, total=100, maxlen=60, H=4, Hkv=2, d=128,
             idt=BF16, odt=F32, out=A[3], lse=None, ws=A[8], wsb=1 << 40, **kw):
        o = _lib.softmax_options(**kw)
        return lib.la_softmax_attention_varlen(q, k, v, cu, nseq, total, maxlen, H, Hkv, d, idt,
                                               odt, out, lse, ctypes.byref(o), ws, wsb, None)

    assert call(q=None) == INVALID
    assert call(cu=None) == INVALID
    assert call(out=None) == INVALID
    assert call(q=ctypes.c_void_p(0x10000008)) == INVALID          # misaligned
    assert call(nseq=0) == INVALID
    assert call(total=-1) == INVALID
    assert call(maxlen=101) == INVALID                             # above total_T
    assert call(maxlen=0) == INVALID                               # tokens but no length bound
    assert call(Hkv=3) == INVALID                                  # does not divide H
    assert call(H=0) == INVALID
    assert call(d=64) == UNSUPPORTED
    assert call(idt=F32) == UNSUPPORTED
    assert call(idt=7) == INVALID
    assert call(H=1 << 14, Hkv=1) == UNSUPPORTED                   # H*d past 2^20
    assert call(rotary_dim=3) == INVALID
    assert call(rotary_dim=130) == INVALID
    assert call(rotary_dim=24) == UNSUPPORTED                      # not a multiple of 16
    assert call(rope_base=0.0) == INVALID
    assert call(rope_base=float("inf")) == INVALID
    assert call(scale=-1.0) == INVALID
    assert call(precision=3) == INVALID
    assert call(precision=-1) == INVALID
    assert call(out=A[0]) == INVALID                               # out overlaps q
    assert call(lse=ctypes.c_void_p(A[3].value + 64)) == INVALID   # lse overlaps out
    assert call(ws=None) == INVALID
    assert call(ws=ctypes.c_void_p(0x10000010)) == INVALID         # workspace not 256-aligned
    need = lib.la_softmax_workspace_bytes(2, 100, 60, 4, 2, 128, BF16, F32,
                                          ctypes.byref(_lib.softmax_options()))
    assert call(wsb=need - 1) == WS_SMALL
    # an empty batch is accepted with no pointers and launches nothing
    assert call(q=None, k=None, v=None, cu=None, out=None, total=0, maxlen=0, ws=None, wsb=0) == 0


def test_projection_rejects_bad_arguments(lib):
    """la_qkvx_projection's host checks (no call reaches the device)."""
    def call(h=A[0], w=A[1], q=A[2], k=A[3], v=A[4], xg=A[5], T=300, K=6144, F=1024, odt=BF16,
             o=None):
        o = o or _lib.proj_options()
        return lib.la_qkvx_projection(h, w, q, k, v, xg, T, K, F, odt, ctypes.byref(o), None)

    o = lib.la_proj_default_options()
    assert o.featurize == 1 and o.n_timing == 0
    assert call(T=0) == _lib.LA_OK                       # nothing to do
    assert call(h=None) == INVALID
    assert call(q=None) == INVALID
    assert call(T=-1) == INVALID
    assert call(K=100) == UNSUPPORTED                    # not a multiple of 64
    assert call(F=1000) == UNSUPPORTED                   # not a multiple of 256
    assert call(K=0) == INVALID
    assert call(F=1 << 21) == INVALID
    assert call(odt=7) == INVALID
    assert call(q=ctypes.c_void_p(0x10000008)) == INVALID  # misaligned
    assert call(q=A[0]) == INVALID                       # output overlaps the input
    assert call(k=A[2]) == INVALID                       # outputs overlap each other
    bad = _lib.proj_options()
    bad.featurize = 2
    assert call(o=bad) == INVALID
    # more output tiles than the kernel indexes: T = 2^31 - 1 tokens, 4 x 2^20 features
    far = [ctypes.c_void_p(0x7F0000000000 + (i << 53)) for i in range(4)]
    assert call(T=(1 << 31) - 1, K=64, F=1 << 20, q=far[0], k=far[1], v=far[2],
                xg=far[3]) == UNSUPPORTED



def test_out_projection_rejects_bad_arguments(lib):
    """la_out_projection's host checks (no call reaches the device)."""
    def call(y=A[0], w=A[1], out=A[2], T=300, K=1024, N=6144, odt=BF16, o=None):
        o = o or _lib.proj_options(False)
        return lib.la_out_projection(y, w, out, T, K, N, odt, ctypes.byref(o), None)

    assert call(T=0) == _lib.LA_OK                       # nothing to do
    assert call(y=None) == INVALID
    assert call(w=None) == INVALID
    assert call(out=None) == INVALID
    assert call(T=-1) == INVALID
    assert call(K=100) == UNSUPPORTED                    # not a multiple of 64
    assert call(N=1000) == UNSUPPORTED                   # not a multiple of 256
    assert call(K=0) == INVALID
    assert call(N=1 << 21) == INVALID
    assert call(odt=7) == INVALID
    assert call(out=ctypes.c_void_p(0x30000008)) == INVALID  # misaligned
    assert call(out=A[0]) == INVALID                     # output overlaps the input
    assert call(out=ctypes.c_void_p(A[1].value + 4096)) == INVALID  # ... or the weight
    timed = _lib.proj_options(False)
    timed.n_timing = 1                                   # events asked for, none given
    assert call(o=timed) == INVALID
    # more output tiles than the kernel indexes: T = 2^31 - 1 tokens, N = 2^20
    far = ctypes.c_void_p(0x7F0000000000)
    assert call(T=(1 << 31) - 1, K=64, N=1 << 20, out=far) == UNSUPPORTED

def test_projection_bindings_check_operands():
    """The Python entry points refuse operands the C ABI would misread (a
    float32 tensor where bf16 bytes are expected) or host tensors, before any
    call into the library."""
    from linear_attention_long_amd import api

    with pytest.raises(TypeError):
        api.la_out_projection(torch.zeros((4, 64)), torch.zeros((256, 64), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        api.la_qkvx_projection(torch.zeros((4, 64), dtype=torch.bfloat16), torch.zeros((1024, 64)), 256)
    with pytest.raises(ValueError):  # bf16 but on the host
        api.la_out_projection(torch.zeros((4, 64), dtype=torch.bfloat16),
                              torch.zeros((256, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):  # width mismatch
        api.la_out_projection(torch.zeros((4, 64), dtype=torch.bfloat16),
                              torch.zeros((256, 128), dtype=torch.bfloat16))
