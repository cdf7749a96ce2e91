"""Decode step (one token per session) on the GPU against the fp64 oracle."""
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, TOL_BF16_OUT, TOL_F32, dev, close

pytestmark = pytest.mark.gpu


def _decode_case(B, H, Dk, Dv, qkv_dtype, seed, shift=1.0):
    inp = synth.make_dense(B, 1, H, Dk, Dv, seed=seed, qkv_dtype=qkv_dtype, shift=shift,
                           state_std=0.02)
    return inp


def test_decode_b64_h96_d128():
    """Decode workload: 64 sessions x 96 heads x 128 x 128 fp32 state (402,653,184 B)."""
    d = dev()
    w = synth.WORKLOADS["decode_b64"]
    inp = _decode_case(w["B"], w["H"], w["D"], w["D"], w["qkv_dtype"], w["seed"])
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    state = inp.state.to(d)
    o = kda.decode_step(inp.q[:, 0].to(d), inp.k[:, 0].to(d), inp.v[:, 0].to(d),
                        inp.alpha[:, 0].to(d), inp.beta[:, 0].to(d), state)
    torch.cuda.synchronize()
    close(o, o_ref[:, 0], TOL_BF16, "step")
    close(state, s_ref, TOL_BF16, "state")
    # same call on the same inputs is bitwise reproducible
    state2 = inp.state.to(d)
    o2 = kda.decode_step(inp.q[:, 0].to(d), inp.k[:, 0].to(d), inp.v[:, 0].to(d),
                         inp.alpha[:, 0].to(d), inp.beta[:, 0].to(d), state2)
    assert torch.equal(o, o2) and torch.equal(state, state2)


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("qkv", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
def test_decode_shapes_and_dtypes(Dk, Dv, qkv, odt):
    d = dev()
    inp = _decode_case(3, 5, Dk, Dv, qkv, seed=11 + Dk + Dv)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    state = inp.state.to(d)
    o = kda.decode_step(inp.q[:, 0].to(d), inp.k[:, 0].to(d), inp.v[:, 0].to(d),
                        inp.alpha[:, 0].to(d), inp.beta[:, 0].to(d), state, out_dtype=odt)
    torch.cuda.synchronize()
    tol_s = TOL_F32 if qkv == torch.float32 else TOL_BF16
    tol_o = TOL_BF16_OUT if odt == torch.bfloat16 else tol_s
    close(o.float(), o_ref[:, 0], tol_o, "step")
    close(state, s_ref, tol_s, "state")


def test_decode_replay_matches_token_loop():
    """Decode steps chained over a sequence reproduce the oracle's token loop."""
    d = dev()
    B, T, H, D = 2, 40, 4, 128
    inp = synth.make_dense(B, T, H, D, D, seed=21, state_std=0.02)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    state = inp.state.to(d)
    q, k, v, a, b = (x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
    outs = []
    for t in range(T):
        outs.append(kda.decode_step(q[:, t].contiguous(), k[:, t].contiguous(),
                                    v[:, t].contiguous(), a[:, t].contiguous(),
                                    b[:, t].contiguous(), state))
    o = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_BF16, "tokens")
    close(state, s_ref, TOL_BF16, "state")
