"""Chunked and packed prefill on the GPU against the fp64 oracle and against the
GPU decode step replayed token by token.  bf16 cases run under both prefill
schedules (the fused kernel and the two-pass first pass + state pass), which must
also agree with each other bitwise."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, TOL_BF16_OUT, TOL_F32, close, dev, oracle_heads, to

pytestmark = pytest.mark.gpu


SCHEDULES = ["fused", "two_pass"]


def _run(inp, d, out_dtype=torch.float32, schedule="auto"):
    return kda.prefill_chunked(to(inp.q, d), to(inp.k, d), to(inp.v, d), to(inp.alpha, d),
                               to(inp.beta, d), initial_state=to(inp.state, d),
                               out_dtype=out_dtype, schedule=schedule)


def _solo(inp, i, sl, schedule):
    return kda.prefill_chunked(*(x[:, sl].contiguous() for x in
                                 (inp.q, inp.k, inp.v, inp.alpha, inp.beta)),
                               initial_state=inp.state[i:i + 1].contiguous(), schedule=schedule)


def test_tiny_fp32_full():
    """fp32 workload: B=1, H=2, T=256, d=64, zero initial state; tolerance 1e-5."""
    d = dev()
    w = synth.WORKLOADS["tiny_fp32"]
    inp = synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                           qkv_dtype=w["qkv_dtype"], shift=w["shift"], state_std=None)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta)
    o, s = _run(inp, d)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_F32, "tokens")
    close(s, s_ref, TOL_F32, "state")


@pytest.mark.parametrize("B,T,H,Dk,Dv", [
    (2, 200, 3, 128, 128),   # several chunks and a ragged tail
    (1, 77, 2, 64, 64),
    (1, 130, 2, 128, 64),
    (1, 65, 1, 64, 128),
    (1, 1, 2, 128, 128),
    (1, 64, 2, 128, 128),
    (1, 63, 2, 128, 128),
])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_small_bf16_against_oracle(B, T, H, Dk, Dv, schedule):
    d = dev()
    inp = synth.make_dense(B, T, H, Dk, Dv, seed=100 + T + Dk, state_std=0.02)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    o, s = _run(inp, d, schedule=schedule)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_BF16, "tokens")
    close(s, s_ref, TOL_BF16, "state")


def test_fp32_inputs_dv128_and_bf16_output():
    d = dev()
    inp = synth.make_dense(1, 150, 2, 64, 128, seed=31, qkv_dtype=torch.float32, shift=0.0,
                           state_std=0.02)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    o, s = _run(inp, d)
    close(o, o_ref, TOL_F32, "tokens")
    close(s, s_ref, TOL_F32, "state")
    o, s = _run(inp, d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    close(o.float(), o_ref, TOL_BF16_OUT, "tokens")


@pytest.mark.parametrize("Dv", [128, 64])
def test_fp32_inputs_dk128_token_recurrence(Dv):
    """fp32 q, k, v at Dk = 128 (the token recurrence): dense with a ragged
    tail, in-place state, bf16 output, and packed with empty and one-token
    sequences; fp32 tolerance."""
    d = dev()
    inp = synth.make_dense(2, 64 * 3 + 9, 3, 128, Dv, seed=35 + Dv, qkv_dtype=torch.float32,
                           state_std=0.02)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    o, s = _run(inp, d)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_F32, "tokens")
    close(s, s_ref, TOL_F32, "state")
    st = inp.state.to(d)  # in place
    kda.prefill_chunked(to(inp.q, d), to(inp.k, d), to(inp.v, d), to(inp.alpha, d),
                        to(inp.beta, d), initial_state=st, final_state=st)
    o16, _ = _run(inp, d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    close(st, s_ref, TOL_F32, "state")
    close(o16.float(), o_ref, TOL_BF16_OUT, "tokens")
    lengths = [40, 0, 1, 129]
    pk = synth.make_varlen(lengths, 2, 128, Dv, seed=36, qkv_dtype=torch.float32, device=d)
    o, s = kda.prefill_varlen(pk.q, pk.k, pk.v, pk.alpha, pk.beta, pk.cu_seqlens,
                              initial_state=pk.state)
    torch.cuda.synchronize()
    cu = pk.cu_seqlens.cpu().numpy()
    o_ref, s_ref = oracle.recurrent(pk.q.cpu(), pk.k.cpu(), pk.v.cpu(), pk.alpha.cpu(),
                                    pk.beta.cpu(), cu_seqlens=cu, initial_state=pk.state.cpu())
    close(o, o_ref, TOL_F32, "tokens", cu=cu)
    close(s, s_ref, TOL_F32, "state")
    assert torch.equal(s[1], pk.state[1])


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("kind", ["slow_decay", "alpha_one", "bounded_gate"])
def test_decay_regimes(kind, schedule):
    """Slow decay (mean alpha ~0.97), alpha = 1 (DeltaNet) and the bounded gate
    g = -5 sigmoid(z) of "Kimi K3 的 KDA" section 6: the state carry dominates."""
    d = dev()
    if kind == "slow_decay":
        inp = synth.make_dense(1, 1024, 4, 128, 128, seed=41, shift=-4.0)
    elif kind == "alpha_one":
        inp = synth.make_dense(1, 1024, 4, 128, 128, seed=42, alpha_one=True)
    else:
        inp = synth.make_dense(1, 1024, 4, 128, 128, seed=43)
        g = torch.Generator().manual_seed(44)
        z = torch.randn(inp.alpha.shape, generator=g, dtype=torch.float64)
        inp.alpha = torch.exp(-5.0 * torch.sigmoid(z)).float()
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    o, s = _run(inp, d, schedule=schedule)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_BF16, "tokens")
    close(s, s_ref, TOL_BF16, "state")


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_zero_length_hands_state_through(schedule):
    d = dev()
    s0 = synth.make_state(2, 3, 128, 128, seed=5).to(d)
    e = torch.empty(2, 0, 3, 128, dtype=torch.bfloat16, device=d)
    a = torch.empty(2, 0, 3, 128, dtype=torch.float32, device=d)
    o, s = kda.prefill_chunked(e, e, e, a, torch.empty(2, 0, 3, device=d), initial_state=s0,
                               schedule="fused" if schedule == "fused" else "auto")
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128) and torch.equal(s, s0)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_two_segments_equal_whole(schedule):
    """Prefill in two calls with the state handed over matches one call."""
    d = dev()
    inp = synth.make_dense(1, 300, 2, 128, 128, seed=51)
    o, s = _run(inp, d, schedule=schedule)
    cut = 130
    o1, s1 = kda.prefill_chunked(*(x[:, :cut].contiguous().to(d) for x in
                                   (inp.q, inp.k, inp.v, inp.alpha, inp.beta)),
                                 initial_state=inp.state.to(d), schedule=schedule)
    o2, s2 = kda.prefill_chunked(*(x[:, cut:].contiguous().to(d) for x in
                                   (inp.q, inp.k, inp.v, inp.alpha, inp.beta)),
                                 initial_state=s1, schedule=schedule)
    torch.cuda.synchronize()
    close(torch.cat([o1, o2], 1), o, TOL_BF16, "tokens")
    close(s2, s, TOL_BF16, "state")


def _k3_8k(d):
    w = synth.WORKLOADS["k3_prefill_8k"]
    return synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                            state_std=w["state_std"], device=d)


def test_k3_prefill_8k_all_heads():
    """K3-shaped layer (B=1, H=96, T=8192, d=128) at full size against the oracle
    on every head and token, per (sequence, head) bucket; the fused schedule
    and a second launch are bitwise the two-pass result."""
    d = dev()
    inp = _k3_8k(d)
    o, s = _run(inp, d, schedule="two_pass")
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_heads(inp, list(range(inp.q.shape[2])))
    close(o, o_ref, TOL_BF16, "tokens")
    close(s, s_ref, TOL_BF16, "state")
    del o_ref, s_ref
    o2, s2 = _run(inp, d, schedule="two_pass")
    o3, s3 = _run(inp, d, schedule="fused")
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)
    assert torch.equal(o, o3) and torch.equal(s, s3)


def test_k3_prefill_8k_matches_decode_replay():
    """All 96 heads: chunked prefill (the schedule the library picks for this
    shape) vs the GPU decode step replayed token by token."""
    d = dev()
    inp = _k3_8k(d)
    o, s = _run(inp, d)
    state = inp.state.clone()
    T = inp.q.shape[1]
    orep = torch.empty_like(o)
    for t in range(T):
        kda.decode_step(inp.q[:, t], inp.k[:, t], inp.v[:, t], inp.alpha[:, t], inp.beta[:, t],
                        state, o=orep[:, t])
    torch.cuda.synchronize()
    close(o, orep, TOL_BF16, "tokens")
    close(s, state, TOL_BF16, "state")


def _varlen_case(lengths, H, D, seed, d):
    return synth.make_varlen(lengths, H, D, D, seed=seed, device=d)


def _run_varlen(inp, d, schedule="auto"):
    return kda.prefill_varlen(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.cu_seqlens,
                              initial_state=inp.state, schedule=schedule)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_varlen_edges_and_isolation(schedule):
    """Empty, 1-token, chunk-boundary and ragged sequences in one packed batch; each
    sequence must equal the oracle and, bitwise, its own solo run."""
    d = dev()
    lengths = [0, 1, 63, 64, 65, 200, 7]
    inp = _varlen_case(lengths, 3, 128, seed=61, d=d)
    o, s = _run_varlen(inp, d, schedule)
    torch.cuda.synchronize()
    cu = inp.cu_seqlens.cpu().numpy()
    o_ref, s_ref = oracle.recurrent(inp.q.cpu(), inp.k.cpu(), inp.v.cpu(), inp.alpha.cpu(),
                                    inp.beta.cpu(), cu_seqlens=cu, initial_state=inp.state.cpu())
    close(o, o_ref, TOL_BF16, "tokens", cu=cu)
    close(s, s_ref, TOL_BF16, "state")
    for i in range(len(lengths)):
        sl = slice(int(cu[i]), int(cu[i + 1]))
        oi, si = _solo(inp, i, sl, schedule)
        assert torch.equal(oi, o[:, sl]) and torch.equal(si, s[i:i + 1])


def test_varlen_16_sequences_all_heads():
    """Packed workload: 16 sequences, lengths uniform in [1024, 16384] from the seed,
    H=96, d=128, per-sequence initial / final state.  The oracle runs on every
    head of every sequence (in groups of heads, to bound host memory), compared
    per (sequence, head) bucket; the fused schedule is bitwise the two-pass
    result, and 3 sequences are compared bitwise with solo runs."""
    d = dev()
    w = synth.WORKLOADS["varlen_16"]
    lengths = synth.varlen_lengths(w["N"], w["lo"], w["hi"], seed=w["seed"])
    inp = _varlen_case(lengths, w["H"], w["D"], seed=w["seed"], d=d)
    o, s = _run_varlen(inp, d, "two_pass")
    torch.cuda.synchronize()
    cu = inp.cu_seqlens.cpu().numpy()
    for h0 in range(0, w["H"], 24):
        heads = list(range(h0, min(w["H"], h0 + 24)))
        o_ref, s_ref = oracle_heads(inp, heads, cu=cu)
        close(o[:, :, heads], o_ref, TOL_BF16, "tokens", cu=cu)
        close(s[:, heads], s_ref, TOL_BF16, "state")
        del o_ref, s_ref
    o2, s2 = _run_varlen(inp, d, "fused")
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(s, s2)
    order = np.argsort(lengths)
    for i in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        sl = slice(int(cu[i]), int(cu[i + 1]))
        oi, si = _solo(inp, i, sl, "two_pass")
        assert torch.equal(oi, o[:, sl]) and torch.equal(si, s[i:i + 1])


@pytest.mark.parametrize("B,T,H,Dk,Dv", [
    (2, 200, 3, 128, 128), (1, 77, 2, 64, 64), (1, 130, 2, 128, 64), (1, 300, 1, 64, 128),
])
def test_schedules_agree_bitwise(B, T, H, Dk, Dv):
    """The two schedules compute the same products in the same order."""
    d = dev()
    inp = synth.make_dense(B, T, H, Dk, Dv, seed=300 + T, state_std=0.02)
    for out_dtype in (torch.float32, torch.bfloat16):
        o1, s1 = _run(inp, d, out_dtype, schedule="fused")
        o2, s2 = _run(inp, d, out_dtype, schedule="two_pass")
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
    lengths = [130, 1, 0, 64, 257]
    vin = _varlen_case(lengths, 2, 128, seed=71, d=d)
    o1, s1 = _run_varlen(vin, d, "fused")
    o2, s2 = _run_varlen(vin, d, "two_pass")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_two_pass_workspace_reuse_and_capacity():
    """One caller-owned workspace (its size does not depend on T) serves calls of
    different lengths, and the packed layout holds when every sequence ends in a
    partial chunk."""
    d = dev()
    ws = torch.empty(kda.workspace_size(1, 64, 4, 128, 128), dtype=torch.uint8, device=d)
    for T in (1024, 70, 9000):
        inp = synth.make_dense(1, T, 4, 128, 128, seed=400 + T, state_std=0.02)
        o1, s1 = _run(inp, d, schedule="fused")
        o2, s2 = kda.prefill_chunked(inp.q.to(d), inp.k.to(d), inp.v.to(d), inp.alpha.to(d),
                                     inp.beta.to(d), initial_state=inp.state.to(d),
                                     schedule="two_pass", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
    lengths = [65] * 9 + [1] * 5
    vin = _varlen_case(lengths, 2, 64, seed=72, d=d)
    need = kda._lib.varlen_workspace_size(len(lengths), sum(lengths), 2, 64, 64)
    ws = torch.empty(need, dtype=torch.uint8, device=d)
    o1, s1 = _run_varlen(vin, d, "fused")
    o2, s2 = kda.prefill_varlen(vin.q, vin.k, vin.v, vin.alpha, vin.beta, vin.cu_seqlens,
                                initial_state=vin.state, schedule="two_pass", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_two_pass_windows():
    """Several 8192-token windows: dense sequences longer than a window, packed
    sequences that start, end or lie entirely inside later windows (and empty
    ones among them), state handed over in place or not returned at all.  The
    two-pass result equals the fused kernel bitwise and the oracle within 2e-3."""
    d = dev()
    inp = synth.make_dense(2, 9000, 2, 128, 128, seed=501, state_std=0.02)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    o1, s1 = _run(inp, d, schedule="fused")
    o2, s2 = _run(inp, d, schedule="two_pass")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    close(o2, o_ref, TOL_BF16, "tokens")
    close(s2, s_ref, TOL_BF16, "state")
    # final state written over the initial state, and no final state at all
    st = inp.state.to(d).clone()
    g = [x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
    o3, _ = kda.prefill_chunked(*g, initial_state=st, final_state=st, schedule="two_pass")
    o4, none = kda.prefill_chunked(*g, initial_state=inp.state.to(d), final_state=False,
                                   schedule="two_pass")
    torch.cuda.synchronize()
    assert none is None and torch.equal(st, s1) and torch.equal(o3, o1) and torch.equal(o4, o1)
    lengths = [6000, 0, 2500, 64, 8192, 1, 0, 9000, 130]
    vin = _varlen_case(lengths, 2, 64, seed=73, d=d)
    cu = vin.cu_seqlens.cpu().numpy()
    o_ref, s_ref = oracle.recurrent(vin.q.cpu(), vin.k.cpu(), vin.v.cpu(), vin.alpha.cpu(),
                                    vin.beta.cpu(), cu_seqlens=cu, initial_state=vin.state.cpu())
    o1, s1 = _run_varlen(vin, d, "fused")
    o2, s2 = _run_varlen(vin, d, "two_pass")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    close(o2, o_ref, TOL_BF16, "tokens", cu=cu)
    close(s2, s_ref, TOL_BF16, "state")


def test_two_pass_on_caller_stream_and_in_a_graph():
    """The two-pass schedule (two launches per 8192-token window) on a
    non-default caller stream, and captured in a graph replayed several times
    with eager work between the replays, gives bitwise the eager result."""
    d = dev()
    inp = synth.make_dense(1, 10000, 3, 128, 128, seed=511, state_std=0.02, device=d)
    ref_o, ref_s = _run(inp, d, schedule="fused")
    ws = torch.empty(kda.workspace_size(1, 10000, 3, 128, 128), dtype=torch.uint8, device=d)
    o = torch.empty_like(ref_o)
    fs = torch.empty_like(ref_s)

    def call():
        kda.prefill_chunked(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state,
                            final_state=fs, o=o, schedule="two_pass", workspace=ws)

    side = torch.cuda.Stream(device=d)
    side.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(side):
        for _ in range(2):
            call()
    torch.cuda.current_stream(d).wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(fs, ref_s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        o.zero_()
        fs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(fs, ref_s)
        _run(inp, d, schedule="fused")  # eager work between replays


def _fast_decay(B, T, H, D, seed, qkv_dtype=torch.bfloat16, channel=None):
    """-log alpha ~ N(6, 0.5^2) per token and channel (a 16-token tile decays by
    about e^-96, past fp32's range), or only in one channel with the workloads'
    gate elsewhere: inside (0, 1] but beyond what the factored diagonal tile
    can hold, so every such tile takes the exact path."""
    inp = synth.make_dense(B, T, H, D, D, seed=seed, qkv_dtype=qkv_dtype, state_std=0.02)
    g = torch.Generator().manual_seed(seed + 1)
    fast = torch.exp(-(6.0 + 0.5 * torch.randn(inp.alpha.shape, generator=g,
                                                 dtype=torch.float64))).float()
    if channel is None:
        inp.alpha = fast
    else:
        inp.alpha[..., channel] = fast[..., channel]
    return inp


@pytest.mark.parametrize("channel", [None, 5])
def test_fast_decay_takes_the_exact_tile_path(channel):
    """Both schedules against the oracle per (sequence, head), bitwise against
    each other, and against the GPU decode step replayed token by token."""
    d = dev()
    inp = _fast_decay(1, 1000, 3, 128, seed=810 + (channel or 0), channel=channel)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    res = {}
    for sch in SCHEDULES:
        o, s = _run(inp, d, schedule=sch)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(s).all(), sch
        close(o, o_ref, TOL_BF16, "tokens")
        close(s, s_ref, TOL_BF16, "state")
        res[sch] = (o, s)
    assert torch.equal(res["fused"][0], res["two_pass"][0])
    assert torch.equal(res["fused"][1], res["two_pass"][1])
    q, k, v, a, b = (x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
    state = inp.state.to(d)
    orep = torch.empty_like(res["two_pass"][0])
    for t in range(q.shape[1]):
        kda.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                        a[:, t].contiguous(), b[:, t].contiguous(), state, o=orep[:, t])
    torch.cuda.synchronize()
    close(res["two_pass"][0], orep, TOL_BF16, "tokens")
    close(res["two_pass"][1], state, TOL_BF16, "state")


def test_fast_decay_segmented_packed_and_fp32():
    """The exact tile path under the segmented schedule on packed sequences,
    and in the fp32-input kernel (tolerance 1e-5)."""
    d = dev()
    lengths = [300, 1, 0, 130, 64]
    inp = synth.make_varlen(lengths, 2, 128, 128, seed=820)
    g = torch.Generator().manual_seed(821)
    inp.alpha = torch.exp(-(6.0 + 0.5 * torch.randn(inp.alpha.shape, generator=g,
                                                      dtype=torch.float64))).float()
    cu = inp.cu_seqlens.numpy()
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta, cu_seqlens=cu,
                                    initial_state=inp.state)
    o, s = kda.prefill_segmented(*(x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)),
                                 initial_state=inp.state.to(d), cu_seqlens=inp.cu_seqlens.to(d),
                                 n_segments=3)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_BF16, "tokens", cu=cu)
    close(s, s_ref, TOL_BF16, "state")
    f = _fast_decay(1, 200, 2, 64, seed=830, qkv_dtype=torch.float32)
    o_ref, s_ref = oracle.recurrent(f.q, f.k, f.v, f.alpha, f.beta, initial_state=f.state)
    o, s = _run(f, d)
    torch.cuda.synchronize()
    close(o, o_ref, TOL_F32, "tokens")
    close(s, s_ref, TOL_F32, "state")


def test_bounded_gate_at_its_floor_keeps_the_factored_path():
    """K3's bounded gate at g = g_min = -5 for every token (logits far in the
    saturated range): each 16-token tile decays by e^-80, just inside the
    factored form's range, so no tile is flagged and the result matches."""
    d = dev()
    inp = synth.make_dense(1, 500, 2, 128, 128, seed=840, state_std=0.02)
    z = torch.full(inp.alpha.shape, 60.0)
    a_log = torch.zeros(2)
    alpha = oracle.gate_alpha("bounded", z.numpy(), z.shape, a_log=a_log.numpy())
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta,
                                    initial_state=inp.state)
    for sch in SCHEDULES:
        o, s = kda.prefill_chunked(*(x.to(d) for x in (inp.q, inp.k, inp.v)), z.to(d),
                                   inp.beta.to(d), initial_state=inp.state.to(d), schedule=sch,
                                   gate="bounded", a_log=a_log.to(d))
        torch.cuda.synchronize()
        close(o, o_ref, TOL_BF16, "tokens")
        close(s, s_ref, TOL_BF16, "state")


@pytest.mark.parametrize("kind", ["alpha_one", "slow_decay", "one_slow_channel"])
def test_long_slow_decay_keeps_w_split(kind):
    """16384 tokens (the longest packed sequence's length) where the state
    barely forgets: alpha = 1 given as a tensor, slow decay (mean alpha ~0.97),
    and the workloads' gate with one channel at alpha = 0.9999.  Chunks where
    some channel keeps half its state keep W of W S split, so the rounding
    does not build up along the sequence; both schedules against the oracle
    (and each other, bitwise)."""
    d = dev()
    if kind == "alpha_one":
        inp = synth.make_dense(1, 16384, 2, 128, 128, seed=850, alpha_one=True)
    elif kind == "slow_decay":
        inp = synth.make_dense(1, 16384, 2, 128, 128, seed=851, shift=-4.0)
    else:
        inp = synth.make_dense(1, 16384, 2, 128, 128, seed=852)
        inp.alpha[..., 77] = 0.9999
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                    initial_state=inp.state)
    res = {}
    for sch in SCHEDULES:
        o, s = _run(inp, d, schedule=sch)
        torch.cuda.synchronize()
        g_o, _ = close(o, o_ref, TOL_BF16, "tokens")
        g_s, _ = close(s, s_ref, TOL_BF16, "state")
        print(f"[{kind} {sch}] rel-L2 o={g_o:.2e} S={g_s:.2e}")
        res[sch] = (o, s)
    assert torch.equal(res["fused"][0], res["two_pass"][0])
    assert torch.equal(res["fused"][1], res["two_pass"][1])
