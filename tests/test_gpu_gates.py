"""The gate parametrizations on the GPU: the log-space gate, K3's bounded gate,
the scalar (gated DeltaNet) gate and no gate (DeltaNet), through the *_gated
entry points, against the fp64 oracle fed the decay the oracle itself forms from
the same gate tensor."""
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, TOL_F32, dev, close

pytestmark = pytest.mark.gpu

KINDS = ["log", "bounded", "scalar", "none"]
SCHEDULES = ["fused", "two_pass"]


def _case(B, T, H, Dk, Dv, kind, seed, qkv_dtype=torch.bfloat16, lengths=None):
    if lengths is None:
        inp = synth.make_dense(B, T, H, Dk, Dv, seed=seed, qkv_dtype=qkv_dtype, state_std=0.02)
    else:
        inp = synth.make_varlen(lengths, H, Dk, Dv, seed=seed, qkv_dtype=qkv_dtype)
    lead = tuple(inp.q.shape[:2])
    gate, a_log = synth.make_gate(kind, lead, H, Dk, seed=seed + 1)
    alpha = oracle.gate_alpha(kind, None if gate is None else gate.numpy(), inp.q.shape,
                              a_log=None if a_log is None else a_log.numpy())
    return inp, gate, a_log, alpha


def _to(x, d):
    return None if x is None else x.to(d)


def _prefill(inp, gate, a_log, kind, d, schedule, out_dtype=torch.float32):
    kw = dict(initial_state=_to(inp.state, d), out_dtype=out_dtype, schedule=schedule,
              gate=kind, a_log=_to(a_log, d))
    if inp.cu_seqlens is None:
        return kda.prefill_chunked(inp.q.to(d), inp.k.to(d), inp.v.to(d), _to(gate, d),
                                   inp.beta.to(d), **kw)
    return kda.prefill_varlen(inp.q.to(d), inp.k.to(d), inp.v.to(d), _to(gate, d),
                              inp.beta.to(d), inp.cu_seqlens.to(d), **kw)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("B,T,H,Dk,Dv", [(2, 333, 3, 128, 128), (1, 150, 2, 64, 64)])
def test_prefill_gates_bf16(kind, B, T, H, Dk, Dv):
    """bf16 prefill with each gate kind; both schedules agree bitwise."""
    d = dev()
    inp, gate, a_log, alpha = _case(B, T, H, Dk, Dv, kind, seed=500 + T)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta,
                                    initial_state=inp.state)
    res = {}
    for sch in SCHEDULES:
        o, s = _prefill(inp, gate, a_log, kind, d, sch)
        torch.cuda.synchronize()
        close(o, o_ref, TOL_BF16, "tokens")
        close(s, s_ref, TOL_BF16, "state")
        res[sch] = (o, s)
    assert torch.equal(res["fused"][0], res["two_pass"][0])
    assert torch.equal(res["fused"][1], res["two_pass"][1])


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("Dk", [64, 128])
def test_prefill_gates_fp32(kind, Dk):
    """fp32 inputs (the fp32 chunk kernel at Dk 64, the token recurrence at
    Dk 128): tolerance 1e-5."""
    d = dev()
    inp, gate, a_log, alpha = _case(1, 150, 2, Dk, 128, kind, seed=610 + Dk,
                                    qkv_dtype=torch.float32)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta,
                                    initial_state=inp.state)
    o, s = _prefill(inp, gate, a_log, kind, d, "auto")
    torch.cuda.synchronize()
    close(o, o_ref, TOL_F32, "tokens")
    close(s, s_ref, TOL_F32, "state")


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("kind", ["bounded", "scalar"])
def test_varlen_gates(kind, schedule):
    """Packed batch with empty, short and ragged sequences under a gate."""
    d = dev()
    lengths = [130, 1, 0, 64, 257, 20]
    inp, gate, a_log, alpha = _case(1, None, 2, 128, 128, kind, seed=640, lengths=lengths)
    cu = inp.cu_seqlens.numpy()
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta, cu_seqlens=cu,
                                    initial_state=inp.state)
    o, s = _prefill(inp, gate, a_log, kind, d, schedule)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_BF16, "tokens", cu=cu)
    close(s, s_ref, TOL_BF16, "state")


def test_gates_reduce_to_alpha_bitwise():
    """The kernels form the same fp32 alpha either way: a scalar gate equals the
    per-channel alpha that repeats it, bitwise, on the prefill (both schedules)
    and the decode step, and so does no gate against alpha = 1 on the decode
    step.  On the prefill the gate without decay keeps W of W S split (the
    state never forgets, so a single rounding of W would accumulate), which
    alpha = 1 given as a tensor does not: there the no-decay result is held to
    a tighter bar against the oracle."""
    d = dev()
    B, T, H, D = 1, 200, 3, 128
    inp = synth.make_dense(B, T, H, D, D, seed=650, state_std=0.02)
    sc, _ = synth.make_gate("scalar", (B, T), H, D, seed=651)
    full = sc[..., None].expand(B, T, H, D).contiguous()
    ones = torch.ones(B, T, H, D)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, ones.numpy(), inp.beta,
                                    initial_state=inp.state)
    for sch in SCHEDULES:
        o1, s1 = _prefill(inp, sc, None, "scalar", d, sch)
        inp_a = synth.KdaInputs(inp.q, inp.k, inp.v, full, inp.beta, inp.state)
        o2, s2 = _prefill(inp_a, full, None, "alpha", d, sch)
        o3, s3 = _prefill(inp, None, None, "none", d, sch)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2), sch
        close(o3, o_ref, 1e-4, "tokens")
        close(s3, s_ref, 1e-4, "state")
    for g1, k1, g2 in ((sc, "scalar", full), (None, "none", ones)):
        st1, st2 = inp.state.to(d), inp.state.to(d)
        o1 = kda.decode_step(inp.q[:, 0].to(d), inp.k[:, 0].to(d), inp.v[:, 0].to(d),
                             None if g1 is None else g1[:, 0].to(d), inp.beta[:, 0].to(d), st1,
                             gate=k1)
        o2 = kda.decode_step(inp.q[:, 0].to(d), inp.k[:, 0].to(d), inp.v[:, 0].to(d),
                             g2[:, 0].contiguous().to(d), inp.beta[:, 0].to(d), st2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(st1, st2), k1


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("qkv", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128)])
def test_decode_gates(kind, qkv, Dk, Dv):
    d = dev()
    B, H = 4, 3
    inp, gate, a_log, alpha = _case(B, 1, H, Dk, Dv, kind, seed=700 + Dk, qkv_dtype=qkv)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta,
                                    initial_state=inp.state)
    state = inp.state.to(d)
    o = kda.decode_step(inp.q[:, 0].to(d), inp.k[:, 0].to(d), inp.v[:, 0].to(d),
                        None if gate is None else gate[:, 0].contiguous().to(d),
                        inp.beta[:, 0].to(d), state, gate=kind, a_log=_to(a_log, d))
    torch.cuda.synchronize()
    tol = TOL_F32 if qkv == torch.float32 else TOL_BF16
    close(o, o_ref[:, 0], tol, "step")
    close(state, s_ref, tol, "state")


def test_k3_prefill_8k_bounded_gate_sampled_heads():
    """K3-shaped layer (B=1, H=96, T=8192, d=128) fed its bounded gate (logits and
    per-head A, g_min = -5): two-pass schedule, oracle on 6 heads."""
    d = dev()
    w = synth.WORKLOADS["k3_prefill_8k"]
    B, T, H, D = w["B"], w["T"], w["H"], w["D"]
    inp = synth.make_dense(B, T, H, D, D, seed=w["seed"], state_std=w["state_std"], device=d)
    z, a_log = synth.make_gate("bounded", (B, T), H, D, seed=w["seed"], device=d)
    o, s = kda.prefill_chunked(inp.q, inp.k, inp.v, z, inp.beta, initial_state=inp.state,
                               schedule="two_pass", gate="bounded", a_log=a_log)
    torch.cuda.synchronize()
    heads = [2, 19, 38, 57, 76, 93]
    zc = z[:, :, heads].cpu().numpy()
    alpha = oracle.gate_alpha("bounded", zc, zc.shape, a_log=a_log[heads].cpu().numpy())
    sel = lambda t: t[:, :, heads].cpu()  # noqa: E731
    o_ref, s_ref = oracle.recurrent(sel(inp.q), sel(inp.k), sel(inp.v), alpha, sel(inp.beta),
                                    initial_state=inp.state[:, heads].cpu())
    close(o[:, :, heads], o_ref, TOL_BF16, "tokens")
    close(s[:, heads], s_ref, TOL_BF16, "state")
