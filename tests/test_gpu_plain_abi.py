"""The plain C entry points (kda_prefill_chunked, kda_prefill_varlen,
kda_decode_step: the decay as an alpha tensor) called through ctypes on real
data, against the fp64 oracle, and bitwise against their gated forms (which the
Python binding calls) with the same alpha."""
import ctypes

import numpy as np
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, TOL_F32, close, dev

pytestmark = pytest.mark.gpu

KDA_F32, KDA_BF16 = 0, 1


def _p(x):
    return ctypes.c_void_p(0 if x is None else x.data_ptr())


def _dt(x):
    return KDA_BF16 if x.dtype == torch.bfloat16 else KDA_F32


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(status):
    lib = kda.load()
    assert status == 0, lib.kda_last_error_message().decode()


@pytest.mark.parametrize("B,T,H,Dk,Dv,qkv", [
    (2, 64 * 3 + 17, 2, 128, 128, torch.bfloat16),
    (1, 150, 3, 64, 128, torch.bfloat16),
    (2, 64 * 2 + 5, 2, 64, 64, torch.float32),
    (2, 64 * 2 + 5, 2, 128, 128, torch.float32),
])
@pytest.mark.parametrize("two_pass", [False, True])
def test_prefill_chunked(B, T, H, Dk, Dv, qkv, two_pass):
    if two_pass and qkv == torch.float32:
        pytest.skip("the two-pass schedule takes bf16 q, k, v")
    d = dev()
    lib = kda.load()
    inp = synth.make_dense(B, T, H, Dk, Dv, seed=2100 + T + Dk, qkv_dtype=qkv, state_std=0.02)
    q, k, v, a, b, s0 = (x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.state))
    o = torch.empty(B, T, H, Dv, dtype=torch.float32, device=d)
    s = torch.empty_like(s0)
    ws_bytes = lib.kda_prefill_workspace_size(B, T, H, Dk, Dv, 64) if two_pass else 0
    assert not two_pass or ws_bytes > 0
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=d) if two_pass else None
    _ok(lib.kda_prefill_chunked(_p(q), _p(k), _p(v), _dt(q), _p(a), _p(b), _p(s0), _p(s), _p(o),
                                KDA_F32, B, T, H, Dk, Dv, 64, _p(ws), ctypes.c_size_t(ws_bytes),
                                _stream()))
    sched = "two_pass" if two_pass else "fused"
    o2, s2 = kda.prefill_chunked(q, k, v, a, b, initial_state=s0, schedule=sched, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)  # the gated form with KDA_GATE_ALPHA
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state)
    tol = TOL_F32 if qkv == torch.float32 else TOL_BF16
    close(o, o_ref, tol, "tokens")
    close(s, s_ref, tol, "state")


@pytest.mark.parametrize("two_pass", [False, True])
def test_prefill_varlen(two_pass):
    d = dev()
    lib = kda.load()
    lengths = [130, 0, 1, 64, 200]
    N, H, D = len(lengths), 2, 128
    tot = sum(lengths)
    inp = synth.make_dense(1, tot, H, D, D, seed=2200, state_std=None)
    s0 = synth.make_state(N, H, D, D, seed=2201).to(d)
    q, k, v, a, b = (x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu = torch.tensor(cu_np, device=d)
    o = torch.empty(1, tot, H, D, dtype=torch.float32, device=d)
    s = torch.empty_like(s0)
    ws_bytes = lib.kda_prefill_varlen_workspace_size(N, tot, H, D, D, 64) if two_pass else 0
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=d) if two_pass else None
    _ok(lib.kda_prefill_varlen(_p(q), _p(k), _p(v), KDA_BF16, _p(a), _p(b), _p(cu), N, tot, _p(s0),
                               _p(s), _p(o), KDA_F32, H, D, D, 64, _p(ws), ctypes.c_size_t(ws_bytes),
                               _stream()))
    sched = "two_pass" if two_pass else "fused"
    o2, s2 = kda.prefill_varlen(q, k, v, a, b, cu, initial_state=s0, schedule=sched, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta, cu_seqlens=cu_np,
                                    initial_state=s0.cpu())
    close(o, o_ref, TOL_BF16, "tokens", cu=cu_np)
    close(s, s_ref, TOL_BF16, "state")
    assert torch.equal(s[1], s0[1])  # the empty sequence hands its state through


@pytest.mark.parametrize("qkv,Dk,Dv", [(torch.bfloat16, 128, 128), (torch.float32, 128, 64),
                                       (torch.bfloat16, 64, 128)])
def test_decode_step(qkv, Dk, Dv):
    d = dev()
    lib = kda.load()
    B, H = 5, 3
    inp = synth.make_dense(B, 1, H, Dk, Dv, seed=2300 + Dk + Dv, qkv_dtype=qkv, state_std=0.02)
    q, k, v, a, b = (x[:, 0].contiguous().to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
    st = inp.state.to(d)
    st2 = st.clone()
    o = torch.empty(B, H, Dv, dtype=torch.float32, device=d)
    _ok(lib.kda_decode_step(_p(q), _p(k), _p(v), _dt(q), _p(a), _p(b), _p(st), _p(o), KDA_F32,
                            B, H, Dk, Dv, _stream()))
    o2 = kda.decode_step(q, k, v, a, b, st2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(st, st2)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state)
    tol = TOL_F32 if qkv == torch.float32 else TOL_BF16
    close(o[:, None], o_ref, tol, "tokens")
    close(st, s_ref, tol, "state")


def test_plain_entry_points_report_argument_errors():
    """A bad argument comes back as KDA_ERR_INVALID_ARGUMENT with a message,
    before anything is launched."""
    d = dev()
    lib = kda.load()
    x = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16, device=d)
    a = torch.ones(1, 64, 1, 128, dtype=torch.float32, device=d)
    b = torch.zeros(1, 64, 1, dtype=torch.float32, device=d)
    o = torch.empty(1, 64, 1, 128, dtype=torch.float32, device=d)
    st = lib.kda_prefill_chunked(_p(x), None, _p(x), KDA_BF16, _p(a), _p(b), None, None, _p(o),
                                 KDA_F32, 1, 64, 1, 128, 128, 64, None, ctypes.c_size_t(0), _stream())
    assert st == 1 and lib.kda_last_error_message().decode()
    st = lib.kda_prefill_chunked(_p(x), _p(x), _p(x), KDA_BF16, _p(a), _p(b), None, None, _p(o),
                                 KDA_F32, 1, 64, 1, 128, 128, 32, None, ctypes.c_size_t(0), _stream())
    assert st == 2  # chunk 32: not built
