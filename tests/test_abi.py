"""Host-side checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments before launching anything.  None of
these calls reaches the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

F32, BF16 = 0, 1
OK, INVALID, UNSUPPORTED = 0, 1, 2
FAKE = 0x10000  # an aligned non-null address; never dereferenced by these calls
# distinct fake tensors, 4 GiB apart: the entry points reject an output that
# overlaps an input, so every argument gets an address range of its own
AT = [FAKE + (i << 32) for i in range(1, 40)]


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = kda.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert getattr(lib, n) is not None
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_status_strings():
    lib = kda.load()
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(1) == b"KDA_ERR_INVALID_ARGUMENT"
    assert lib.kda_status_string(2) == b"KDA_ERR_UNSUPPORTED"
    assert lib.kda_status_string(3) == b"KDA_ERR_HIP"


def test_workspace_sizes():
    """Two-pass workspace: a chunk table (B + 1 int32), one carried fp32 state per
    (sequence, head), and the operand blocks of one 8192-token window, (128 + B) * H
    of them; each block holds the frames of W, (Gamma*Q), Mqk, Ktil^T, T Diag(b)
    and the chunk's v rows, plus Gamma_C and the chunk's W-split flag, rounded
    to 256 B.  Like the state, it does not depend on T."""
    # frames: W (hi, lo), Gamma*Q (hi; lo of tile 0), Mqk (hi, lo), Ktil^T (hi, lo),
    # T Diag(b) (hi, lo), then the chunk's 64 v rows (Dv / 8 frames of 1 KiB)
    frames = {(128, 128): 4 * 4 * 2 + 4 * 4 + 4 + 16 + 8 * 4 + 16 + 16,
              (64, 64): 4 * 2 * 2 + 4 * 2 + 2 + 16 + 4 * 4 + 16 + 8}
    up = lambda x: -(-x // 256) * 256
    for (dk, dv), f in frames.items():
        blk = up(f * 1024 + dk * 4 + 4)
        for B, H in ((1, 1), (1, 96), (3, 2), (16, 96)):
            want = up((B + 1) * 4) + up(B * H * dk * dv * 4) + (128 + B) * H * blk
            sizes = {kda.workspace_size(B, T, H, dk, dv) for T in (1, 256, 8192, 1 << 20)}
            assert sizes == {want}
            assert {_lib.varlen_workspace_size(B, tot, H, dk, dv) for tot in (B, 129161, 1 << 30)} \
                == {want}
    assert kda.workspace_size(1, 256, 96, 128, 128, chunk=32) == ctypes.c_size_t(-1).value
    assert kda.workspace_size(1, 256, 96, 96, 128) == 0          # no two-pass kernel for Dk = 96
    assert kda.workspace_size(0, 256, 96, 128, 128) == 0         # nothing to do


def test_two_pass_preference():
    lib = kda.load()
    # under-filled device, long sequences: two-pass; many short sequences: fused
    assert lib.kda_prefill_two_pass_preferred(BF16, 1, 8192, 96, 128, 128) == 1
    assert lib.kda_prefill_two_pass_preferred(BF16, 64, 64 * 1024, 96, 128, 128) == 0
    assert lib.kda_prefill_two_pass_preferred(BF16, 1, 128, 96, 128, 128) == 0
    assert lib.kda_prefill_two_pass_preferred(F32, 1, 8192, 2, 64, 64) == 0


def test_segmented_workspace_and_preference():
    """The segmented schedule adds the segments' entry states (n_segments
    states per (sequence, head)) and the summaries [M | b] (n_segments - 1 of
    them, Dk x (Dk + Dv) each) to the two-pass workspace; one segment needs
    nothing more."""
    lib = kda.load()
    up = lambda x: -(-x // 256) * 256
    for dk, dv in ((128, 128), (64, 128), (128, 64), (64, 64)):
        for n, H in ((1, 12), (3, 2)):
            base = kda.workspace_size(n, 256, H, dk, dv)
            assert kda.segmented_workspace_size(n, H, dk, dv, 1) == base
            for ns in (2, 8, 16):
                want = base + up(ns * n * H * dk * dv * 4) + (ns - 1) * n * H * dk * (dk + dv) * 4
                assert kda.segmented_workspace_size(n, H, dk, dv, ns) == want
    bad = ctypes.c_size_t(-1).value
    assert kda.segmented_workspace_size(1, 12, 128, 128, 0) == bad
    assert kda.segmented_workspace_size(1, 12, 128, 128, 17) == bad
    assert lib.kda_prefill_segmented_workspace_size(1, 12, 128, 128, 32, 4) == bad
    assert kda.segmented_workspace_size(1, 12, 96, 128, 4) == 0
    # few (sequence, head) pairs and long sequences: segments, at most 8; many
    # heads, short sequences or fp32 inputs: none (these figures assume 256
    # compute units, the count taken when no device is visible)
    pref = lambda *a: lib.kda_prefill_segments_preferred(*a)
    if not __import__("torch").cuda.is_available():
        assert pref(BF16, 1, 8192, 12, 128, 128) == 6
        assert pref(BF16, 1, 8192, 24, 128, 128) == 3
        assert pref(BF16, 1, 8192, 48, 128, 128) == 2
        assert pref(BF16, 1, 8192, 4, 128, 128) == 8   # capped
        assert pref(BF16, 1, 8192, 12, 64, 128) == 8   # smaller summaries
    assert pref(BF16, 1, 8192, 96, 128, 128) == 1
    assert pref(BF16, 1, 448, 12, 128, 128) == 1  # 7 chunks: under 4 per segment
    assert pref(BF16, 1, 512, 12, 128, 128) == 2  # 8 chunks: two segments of 4
    assert pref(F32, 1, 8192, 12, 64, 64) == 1
    assert 1 <= pref(BF16, 2, 2 * 8192, 12, 128, 128) <= 8


def _segmented(**over):
    a = dict(q=AT[0], k=AT[1], v=AT[2], qd=BF16, cu=None, n=1, T=4096, s0=None, s1=None, o=AT[3],
             od=F32, H=2, Dk=128, Dv=128, chunk=64, ns=4, ws=AT[4], wsb=1 << 31)
    a.update(over)
    g = _lib._Gate(0, AT[5], None, 0.0)
    return kda.load().kda_prefill_segmented(
        a["q"], a["k"], a["v"], a["qd"], ctypes.byref(g), AT[6], a["cu"], a["n"], a["T"], a["s0"],
        a["s1"], a["o"], a["od"], a["H"], a["Dk"], a["Dv"], a["chunk"], a["ns"], a["ws"], a["wsb"],
        None)


@pytest.mark.parametrize("over,expect", [
    (dict(ns=0), INVALID),
    (dict(ns=17), INVALID),
    (dict(ws=None, wsb=0), INVALID),
    (dict(wsb=1024), INVALID),
    (dict(ws=AT[4] + 64), INVALID),
    (dict(qd=F32, Dk=64), UNSUPPORTED),
    (dict(Dk=96), UNSUPPORTED),
    (dict(chunk=32), UNSUPPORTED),
    (dict(cu=AT[7] + 2), INVALID),
    (dict(o=AT[0] + 1024), INVALID),      # o overlaps q
    (dict(s0=AT[8], s1=AT[8] + 256), INVALID),  # final state overlaps the initial one
    (dict(s0=AT[8], s1=AT[8], T=0, ws=None, wsb=0, n=0), OK),  # in place is allowed
    (dict(n=-1), INVALID),
    (dict(n=0, q=None, k=None, v=None, o=None, ws=None, wsb=0), OK),
    (dict(T=0, ws=None, wsb=0), OK),  # no tokens and no final state: nothing to do
])
def test_segmented_validation(over, expect):
    assert _segmented(**over) == expect
    if expect != OK:
        assert len(kda.load().kda_last_error_message()) > 0


def _layer(**over):
    a = dict(xq=AT[0], xk=AT[1], xv=AT[2], xd=BF16, taps=AT[3], st=None, so=None, ns=1, T=256,
             o=AT[4], y=AT[4], yd=F32, g=AT[5], w=AT[6], eps=1e-5, ws=AT[7], wsb=1 << 31, H=2,
             Dk=128, Dv=128, chunk=64, beta=AT[8])
    a.update(over)
    c = _lib._Conv(a["taps"], a["taps"] + (1 << 20), a["taps"] + (2 << 20), 1e-6)
    gt = _lib._Gate(0, AT[9], None, 0.0)
    og = _lib._OutGate(a["g"], a["w"], a["eps"])
    return kda.load().kda_prefill_layer(
        a["xq"], a["xk"], a["xv"], a["xd"], ctypes.byref(c), a["st"], a["so"], ctypes.byref(gt),
        a["beta"], None, 1, a["T"], None, None, a["o"], ctypes.byref(og), a["y"], a["yd"], a["H"],
        a["Dk"], a["Dv"], a["chunk"], a["ns"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,expect", [
    (dict(xd=F32), UNSUPPORTED),
    (dict(taps=AT[3] + 4), INVALID),      # taps need 16-byte alignment here
    (dict(st=AT[10], so=AT[10]), INVALID),  # conv state out aliasing in
    (dict(st=AT[10], so=AT[10] + 64), INVALID),  # ... or overlapping it
    (dict(eps=0.0), INVALID),
    (dict(g=None), INVALID),
    (dict(y=AT[11] + 8), INVALID),
    (dict(yd=BF16), INVALID),             # y aliasing o needs fp32
    (dict(o=AT[0]), INVALID),             # o is the x_q buffer
    (dict(o=AT[2] + 4096), INVALID),      # o overlaps x_v
    (dict(y=AT[11], yd=BF16, g=AT[11] + 256), INVALID),  # y overlaps g
    (dict(y=AT[4] + 256), INVALID),       # y overlaps o without being it
    (dict(so=AT[10], st=None, xk=AT[10] + 128), INVALID),  # conv state out overlaps x_k
    (dict(ws=None, wsb=0), INVALID),
    (dict(wsb=4096), INVALID),
    (dict(ns=0), INVALID),
    (dict(Dk=96), UNSUPPORTED),
    (dict(chunk=32), UNSUPPORTED),
])
def test_layer_prefill_validation(over, expect):
    assert _layer(**over) == expect
    assert len(kda.load().kda_last_error_message()) > 0


def _prefill(**over):
    a = dict(q=AT[0], k=AT[1], v=AT[2], qd=BF16, alpha=AT[3], beta=AT[4], s0=None, s1=None,
             o=AT[5], od=F32, B=1, T=128, H=2, Dk=128, Dv=128, chunk=64, ws=None, wsb=0)
    a.update(over)
    lib = kda.load()
    return lib.kda_prefill_chunked(a["q"], a["k"], a["v"], a["qd"], a["alpha"], a["beta"],
                                   a["s0"], a["s1"], a["o"], a["od"], a["B"], a["T"], a["H"],
                                   a["Dk"], a["Dv"], a["chunk"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,expect", [
    (dict(q=None), INVALID),
    (dict(beta=None), INVALID),
    (dict(o=AT[5] + 2), INVALID),
    (dict(q=AT[0] + 1), INVALID),
    (dict(alpha=AT[3] + 8), INVALID),
    (dict(s0=AT[6] + 8), INVALID),
    (dict(o=AT[1] + 512), INVALID),       # o overlaps k
    (dict(o=AT[4]), INVALID),             # o is beta
    (dict(s1=AT[3] + 1024), INVALID),     # final state overlaps alpha
    (dict(s1=AT[5] + 4096), INVALID),     # final state overlaps o
    (dict(H=0), INVALID),
    (dict(T=-1), INVALID),
    (dict(qd=7), INVALID),
    (dict(chunk=32), UNSUPPORTED),
    (dict(Dk=96), UNSUPPORTED),
    (dict(Dv=256), UNSUPPORTED),
    (dict(qd=F32, Dk=128, q=AT[0] + 4), INVALID),  # fp32 at Dk 128: 16-byte loads
    (dict(B=0), OK),
    (dict(ws=AT[7] + 64, wsb=1 << 30), INVALID),
    (dict(ws=AT[5] - 4096, wsb=1 << 20), INVALID),  # workspace overlaps o
])
def test_prefill_argument_validation(over, expect):
    assert _prefill(**over) == expect
    if expect != OK:
        assert len(kda.load().kda_last_error_message()) > 0


def test_varlen_and_decode_validation():
    lib = kda.load()
    # varlen: missing cu_seqlens
    assert lib.kda_prefill_varlen(AT[0], AT[1], AT[2], BF16, AT[3], AT[4], None, 4, 100, None,
                                  None, AT[5], F32, 2, 128, 128, 64, None, 0, None) == INVALID
    # varlen: o overlapping cu_seqlens
    assert lib.kda_prefill_varlen(AT[0], AT[1], AT[2], BF16, AT[3], AT[4], AT[5], 4, 100, None,
                                  None, AT[5], F32, 2, 128, 128, 64, None, 0, None) == INVALID
    # varlen: N == 0 is a no-op
    assert lib.kda_prefill_varlen(None, None, None, BF16, None, None, None, 0, 0, None, None,
                                  None, F32, 2, 128, 128, 64, None, 0, None) == OK
    # decode: missing state, bad head dim, misaligned input, empty batch
    assert lib.kda_decode_step(FAKE, FAKE, FAKE, BF16, FAKE, FAKE, None, FAKE, F32, 4, 2, 128,
                               128, None) == INVALID
    assert lib.kda_decode_step(FAKE, FAKE, FAKE, BF16, FAKE, FAKE, FAKE, FAKE, F32, 4, 2, 96,
                               128, None) == UNSUPPORTED
    assert lib.kda_decode_step(FAKE + 1, FAKE, FAKE, BF16, FAKE, FAKE, FAKE, FAKE, F32, 4, 2, 128,
                               128, None) == INVALID
    assert lib.kda_decode_step(FAKE, FAKE + 8, FAKE, BF16, FAKE, FAKE, FAKE, FAKE, F32, 4, 2, 128,
                               128, None) == INVALID  # 16-byte alignment
    assert lib.kda_decode_step(None, None, None, BF16, None, None, None, None, F32, 0, 2, 128,
                               128, None) == OK


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        kda.prefill_chunked(q, q, q, q, torch.zeros(1, 4, 1))


def _gated(kind, gate=FAKE, a_log=None, g_min=0.0, null_desc=False, entry="chunked", **over):
    lib = kda.load()
    g = _lib._Gate(kind, gate, a_log, g_min)
    gp = None if null_desc else ctypes.byref(g)
    a = dict(qd=BF16, chunk=64, Dk=128)
    a.update(over)
    if entry == "chunked":
        return lib.kda_prefill_chunked_gated(AT[20], AT[21], AT[22], a["qd"], gp, AT[23], None,
                                             None, AT[24], F32, 1, 128, 2, a["Dk"], 128,
                                             a["chunk"], None, 0, None)
    if entry == "varlen":
        return lib.kda_prefill_varlen_gated(AT[20], AT[21], AT[22], a["qd"], gp, AT[23], AT[25],
                                            1, 128, None, None, AT[24], F32, 2, a["Dk"], 128,
                                            a["chunk"], None, 0, None)
    return lib.kda_decode_step_gated(FAKE, FAKE, FAKE, a["qd"], gp, FAKE, FAKE, FAKE, F32, 4, 2,
                                     a["Dk"], 128, None)


ALPHA, LOG, BOUNDED, SCALAR, NONE = (_lib.GATES[n] for n in
                                     ("alpha", "log", "bounded", "scalar", "none"))


@pytest.mark.parametrize("entry", ["chunked", "varlen", "decode"])
@pytest.mark.parametrize("args,expect", [
    (dict(kind=ALPHA, null_desc=True), INVALID),          # no descriptor
    (dict(kind=9), INVALID),                              # unknown kind
    (dict(kind=-1), INVALID),
    (dict(kind=LOG, gate=None), INVALID),                 # tensor missing
    (dict(kind=SCALAR, gate=None), INVALID),
    (dict(kind=BOUNDED, a_log=None, g_min=-5.0), INVALID),
    (dict(kind=BOUNDED, a_log=FAKE + 2, g_min=-5.0), INVALID),
    (dict(kind=BOUNDED, a_log=FAKE, g_min=-5.5), INVALID),  # bound outside [-5, 0)
    (dict(kind=BOUNDED, a_log=FAKE, g_min=0.0), INVALID),
    (dict(kind=BOUNDED, a_log=FAKE, g_min=float("nan")), INVALID),
    (dict(kind=ALPHA, gate=FAKE + 2), INVALID),           # not even 4-byte aligned
    # accepted descriptors, stopped by an unsupported shape before any launch
    (dict(kind=NONE, gate=None, Dk=96), UNSUPPORTED),
    (dict(kind=SCALAR, gate=FAKE + 4, Dk=96), UNSUPPORTED),
    (dict(kind=BOUNDED, a_log=FAKE + 4, g_min=-5.0, Dk=96), UNSUPPORTED),
    (dict(kind=BOUNDED, a_log=FAKE, g_min=-0.5, Dk=96), UNSUPPORTED),
])
def test_gate_validation(entry, args, expect):
    assert _gated(entry=entry, **args) == expect
    assert len(kda.load().kda_last_error_message()) > 0


def test_gate_alignment_per_kind():
    """bf16 prefill and the decode calls read a per-channel gate with 16-byte
    loads; a scalar gate, and the fp32 prefill, need only 4-byte alignment."""
    for kind in (ALPHA, LOG):
        assert _gated(kind=kind, gate=FAKE + 8) == INVALID
        assert _gated(kind=kind, gate=FAKE + 8, entry="varlen") == INVALID
        assert _gated(kind=kind, gate=FAKE + 8, entry="decode") == INVALID
        assert _gated(kind=kind, gate=FAKE + 8, qd=F32, Dk=96) == UNSUPPORTED
    assert _gated(kind=SCALAR, gate=FAKE + 4, entry="decode", Dk=96) == UNSUPPORTED
    assert _gated(kind=BOUNDED, gate=FAKE + 8, a_log=FAKE, g_min=-5.0) == INVALID
    assert _gated(kind=SCALAR, gate=FAKE + 4, chunk=32) == UNSUPPORTED


def test_verify_and_commit_validation():
    lib = kda.load()
    g = _lib._Gate(ALPHA, FAKE, None, 0.0)
    gp = ctypes.byref(g)

    def verify(**o):
        a = dict(q=FAKE, k=FAKE, v=FAKE, qd=BF16, beta=FAKE, st=FAKE, o=FAKE, od=F32, B=2, N=4,
                 H=2, Dk=128, Dv=128, gp=gp)
        a.update(o)
        return lib.kda_decode_verify(a["q"], a["k"], a["v"], a["qd"], a["gp"], a["beta"],
                                     a["st"], a["o"], a["od"], a["B"], a["N"], a["H"], a["Dk"],
                                     a["Dv"], None)

    def commit(**o):
        a = dict(k=FAKE, v=FAKE, qd=BF16, beta=FAKE, n=FAKE, st=FAKE, B=2, N=4, H=2, Dk=128,
                 Dv=128, gp=gp)
        a.update(o)
        return lib.kda_decode_commit(a["k"], a["v"], a["qd"], a["gp"], a["beta"], a["n"],
                                     a["st"], a["B"], a["N"], a["H"], a["Dk"], a["Dv"], None)

    for f in (verify, commit):
        assert f(B=0) == OK and f(N=0) == OK                # nothing to do
        assert f(N=-1) == INVALID and f(B=-1) == INVALID
        assert f(k=None) == INVALID and f(st=None) == INVALID
        assert f(v=FAKE + 8) == INVALID                      # 16-byte alignment
        assert f(st=FAKE + 8) == INVALID
        assert f(gp=None) == INVALID
        assert f(qd=5) == INVALID
        assert f(N=17) == UNSUPPORTED                        # at most 16 tokens
        assert f(Dk=96) == UNSUPPORTED
    assert verify(q=None) == INVALID and verify(o=None) == INVALID
    assert verify(q=FAKE + 8) == INVALID
    assert commit(n=None) == INVALID and commit(n=FAKE + 2) == INVALID


def test_prologue_epilogue_validation():
    lib = kda.load()
    c = _lib._Conv(FAKE, FAKE, FAKE, 1e-6)
    cp = ctypes.byref(c)

    def pro(**o):
        a = dict(xq=FAKE, xk=FAKE + 0x100, xv=FAKE + 0x200, dt=BF16, cp=cp, si=None, so=None,
                 cu=None, N=2, T=8, H=2, Dk=128, Dv=128, q=FAKE + 0x300, k=FAKE + 0x400,
                 v=FAKE + 0x500)
        a.update(o)
        return lib.kda_prologue(a["xq"], a["xk"], a["xv"], a["dt"], a["cp"], a["si"], a["so"],
                                a["cu"], a["N"], a["T"], a["H"], a["Dk"], a["Dv"], a["q"],
                                a["k"], a["v"], None)

    assert pro(N=0) == OK
    assert pro(cp=None) == INVALID
    assert pro(xq=None) == INVALID and pro(v=None) == INVALID
    assert pro(xk=FAKE + 8) == INVALID                      # 16-byte alignment
    assert pro(q=FAKE) == INVALID                           # output aliases x_q
    assert pro(si=FAKE + 0x600, so=FAKE + 0x600) == INVALID  # states alias
    far = lambda i: FAKE + (i << 32)  # noqa: E731
    sep = dict(xq=far(1), xk=far(2), xv=far(3), q=far(4), k=far(5), v=far(6))
    for o, i in (("v", "xq"), ("v", "xk"), ("q", "xv"), ("k", "xv"), ("q", "xk"), ("k", "xq")):
        over = dict(sep)
        over[o] = sep[i] + 256  # overlapping, not equal
        assert pro(**over) == INVALID, (o, i)
    assert pro(**dict(sep, q=far(5) + 16)) == INVALID       # two outputs overlap
    assert pro(**dict(sep, so=far(7), si=None, xv=far(7) + 64)) == INVALID
    c2 = _lib._Conv(far(8), far(8) + (1 << 20), far(8) + (2 << 20), 1e-6)
    assert pro(**dict(sep, cp=ctypes.byref(c2), so=far(8) + 2048)) == INVALID  # taps
    assert pro(**dict(sep, cp=ctypes.byref(c2), Dk=96)) == UNSUPPORTED  # no overlap
    assert pro(dt=9) == INVALID and pro(H=0) == INVALID
    assert pro(Dk=96) == UNSUPPORTED
    bad = _lib._Conv(FAKE, None, FAKE, 1e-6)
    assert pro(cp=ctypes.byref(bad)) == INVALID
    zero_eps = _lib._Conv(FAKE, FAKE, FAKE, 0.0)
    assert pro(cp=ctypes.byref(zero_eps)) == INVALID

    def epi(**o):
        a = dict(o=FAKE, od=F32, g=FAKE + 0x100, gd=BF16, w=FAKE + 0x200, eps=1e-5,
                 y=FAKE + 0x300, yd=BF16, tokens=4, H=2, Dv=128)
        a.update(o)
        return lib.kda_epilogue(a["o"], a["od"], a["g"], a["gd"], a["w"], a["eps"], a["y"],
                                a["yd"], a["tokens"], a["H"], a["Dv"], None)

    assert epi(tokens=0) == OK
    assert epi(g=None) == INVALID and epi(w=None) == INVALID
    assert epi(eps=0.0) == INVALID and epi(eps=float("nan")) == INVALID
    assert epi(y=FAKE) == INVALID                           # aliases o with another dtype
    assert epi(o=FAKE + 4) == INVALID
    assert epi(Dv=96) == UNSUPPORTED
