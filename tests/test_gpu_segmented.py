"""The segmented two-pass prefill on the GPU: each window's chunks of a sequence
cut into segments whose affine summaries (M, b) are composed into entry states.
Checked against the fp64 oracle, against the unsegmented two-pass schedule
(bitwise with one segment, within rounding with several), and on packed
batches with empty, short and window-crossing sequences."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, TOL_BF16_OUT, dev, oracle_heads, close

pytestmark = pytest.mark.gpu

# segmented vs unsegmented: the same split-bf16 products associated differently;
# each product is within about 3 * 2^-18 of fp32, so the two differ far below the
# oracle tolerance
TOL_SEG = 2e-4


def _dense(inp, d, n_segments, **kw):
    g = [x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
    return kda.prefill_segmented(*g, initial_state=None if inp.state is None else inp.state.to(d),
                                 n_segments=n_segments, **kw)


def _two_pass(inp, d):
    g = [x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
    return kda.prefill_chunked(*g, initial_state=None if inp.state is None else inp.state.to(d),
                               schedule="two_pass")


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("n_segments", [2, 5, 16])
def test_dense_against_oracle(Dk, Dv, n_segments):
    """Two sequences of 37 chunks and a ragged tail; every segment count leaves
    some segments longer than others."""
    d = dev()
    inp = synth.make_dense(2, 64 * 37 + 13, 2, Dk, Dv, seed=1200 + Dk + Dv + n_segments,
                           state_std=0.02)
    o, s = _dense(inp, d, n_segments)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    close(o, o_ref, TOL_BF16, "tokens")
    close(s, s_ref, TOL_BF16, "state")
    o2, s2 = _two_pass(inp, d)
    torch.cuda.synchronize()
    close(o, o2, TOL_SEG, "tokens")
    close(s, s2, TOL_SEG, "state")


def test_one_segment_is_the_two_pass_schedule_bitwise():
    d = dev()
    inp = synth.make_dense(1, 5000, 3, 128, 128, seed=1210, state_std=0.02)
    o1, s1 = _dense(inp, d, 1)
    o2, s2 = _two_pass(inp, d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("kind", ["log", "bounded", "scalar", "none"])
def test_gates(kind):
    d = dev()
    B, T, H, D = 1, 64 * 20 + 5, 2, 128
    inp = synth.make_dense(B, T, H, D, D, seed=1220, state_std=0.02)
    gate, a_log = synth.make_gate(kind, (B, T), H, D, seed=1221)
    alpha = oracle.gate_alpha(kind, None if gate is None else gate.numpy(), inp.q.shape,
                              a_log=None if a_log is None else a_log.numpy())
    g = [x.to(d) for x in (inp.q, inp.k, inp.v)]
    o, s = kda.prefill_segmented(*g, None if gate is None else gate.to(d), inp.beta.to(d),
                                 initial_state=inp.state.to(d), n_segments=4, gate=kind,
                                 a_log=None if a_log is None else a_log.to(d))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta,
                                    initial_state=inp.state)
    close(o, o_ref, TOL_BF16, "tokens")
    close(s, s_ref, TOL_BF16, "state")


def test_windows_in_place_and_bf16_output():
    """Three 8192-token windows (the carried state enters each window's
    combine), the final state written over the initial one, bf16 output."""
    d = dev()
    inp = synth.make_dense(1, 2 * 8192 + 1500, 2, 128, 128, seed=1230, state_std=0.02)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    st = inp.state.to(d).clone()
    g = [x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
    o, s = kda.prefill_segmented(*g, initial_state=st, final_state=st, n_segments=8,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert s is st
    close(o.float(), o_ref, TOL_BF16_OUT, "tokens")
    close(st, s_ref, TOL_BF16, "state")
    # no final state at all: same outputs
    o2, none = kda.prefill_segmented(*g, initial_state=inp.state.to(d), final_state=False,
                                     n_segments=8, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert none is None and torch.equal(o, o2)


def test_packed_sequences():
    """Empty, one-token, sub-chunk, window-crossing and multi-window sequences
    packed together; segments are cut per sequence and window."""
    d = dev()
    lengths = [6000, 0, 2500, 64, 8192, 1, 0, 9000, 130, 700]
    inp = synth.make_varlen(lengths, 2, 128, 128, seed=1240, device=d)
    cu = inp.cu_seqlens.cpu().numpy()
    o_ref, s_ref = oracle.recurrent(inp.q.cpu(), inp.k.cpu(), inp.v.cpu(), inp.alpha.cpu(),
                                    inp.beta.cpu(), cu_seqlens=cu, initial_state=inp.state.cpu())
    for ns in (3, 16):
        o, s = kda.prefill_segmented(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                     initial_state=inp.state, cu_seqlens=inp.cu_seqlens,
                                     n_segments=ns)
        torch.cuda.synchronize()
        close(o, o_ref, TOL_BF16, "tokens", cu=cu)
        close(s, s_ref, TOL_BF16, "state")
        for i in (1, 6):  # empty sequences hand their state through exactly
            assert torch.equal(s[i], inp.state[i])


def test_workspace_reuse_and_determinism():
    """One workspace for calls of different sizes; a repeated call is bitwise
    identical."""
    d = dev()
    big = kda.segmented_workspace_size(2, 3, 128, 128, 8)
    ws = torch.empty(big, dtype=torch.uint8, device=d)
    a = synth.make_dense(2, 3000, 3, 128, 128, seed=1250, state_std=0.02)
    b = synth.make_dense(1, 900, 2, 128, 128, seed=1251, state_std=0.02)
    oa, sa = _dense(a, d, 8, workspace=ws)
    ob, sb = _dense(b, d, 6, workspace=ws)
    oa2, sa2 = _dense(a, d, 8, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(oa, oa2) and torch.equal(sa, sa2)
    o_ref, s_ref = oracle.recurrent(b.q, b.k, b.v, b.alpha, b.beta, initial_state=b.state)
    close(ob, o_ref, TOL_BF16, "tokens")
    close(sb, s_ref, TOL_BF16, "state")
    with pytest.raises((kda.KdaError, ValueError)):  # the binding checks the size first
        _dense(a, d, 8, workspace=ws[: big - 256])


def test_k3_8k_twelve_heads():
    """One device's share of the 8K layer under an 8-way head split (12 heads,
    T = 8192, d = 128) with the library's segment count: the oracle on 3 heads,
    the unsegmented two-pass schedule on all of them."""
    d = dev()
    w = synth.WORKLOADS["k3_prefill_8k_h12"]
    inp = synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                           state_std=w["state_std"], device=d)
    ns = kda.segments_preferred(torch.bfloat16, 1, w["T"], w["H"], w["D"], w["D"])
    assert ns > 1
    o, s = _dense(inp, d, None)
    o2, s2 = _two_pass(inp, d)
    torch.cuda.synchronize()
    close(o, o2, TOL_SEG, "tokens")
    close(s, s2, TOL_SEG, "state")
    heads = [0, 5, 11]
    o_ref, s_ref = oracle_heads(inp, heads)
    close(o[:, :, heads], o_ref, TOL_BF16, "tokens")
    close(s[:, heads], s_ref, TOL_BF16, "state")


def test_in_a_graph():
    """Two windows of summary, combine and state passes captured in a graph and
    replayed several times, with eager work between the replays: every replay
    gives bitwise the eager result."""
    d = dev()
    inp = synth.make_dense(1, 8192 + 3000, 2, 128, 128, seed=1260, state_std=0.02, device=d)
    g = (inp.q, inp.k, inp.v, inp.alpha, inp.beta)
    ws = torch.empty(kda.segmented_workspace_size(1, 2, 128, 128, 5), dtype=torch.uint8, device=d)
    ref_o, ref_s = kda.prefill_segmented(*g, initial_state=inp.state, n_segments=5, workspace=ws)
    o = torch.empty_like(ref_o)
    fs = torch.empty_like(ref_s)

    def call():
        kda.prefill_segmented(*g, initial_state=inp.state, final_state=fs, o=o, n_segments=5,
                              workspace=ws)

    side = torch.cuda.Stream(device=d)
    side.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream(d).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        o.zero_()
        fs.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(fs, ref_s)
        _dense(synth.make_dense(1, 700, 2, 128, 128, seed=1261, state_std=0.02), d, 3,
               workspace=ws)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
