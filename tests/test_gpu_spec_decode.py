"""Speculative decoding on the GPU: verify (N draft tokens from the state, which
stays untouched) and commit (the accepted prefix folded into the state), against
the fp64 oracle and against N single decode steps (bitwise for the token loop
below four drafts, within fp32 rounding for the chunk form from four on)."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, TOL_BF16_OUT, TOL_F32, dev, close

pytestmark = pytest.mark.gpu


def _case(B, N, H, Dk, Dv, seed, qkv=torch.bfloat16, kind="alpha", device="cpu"):
    inp = synth.make_dense(B, N, H, Dk, Dv, seed=seed, qkv_dtype=qkv, state_std=0.02,
                           device=device)
    if kind == "alpha":
        gate, a_log = inp.alpha, None
    else:
        gate, a_log = synth.make_gate(kind, (B, N), H, Dk, seed=seed + 1, device=device)
    alpha = oracle.gate_alpha(kind, None if gate is None else gate.cpu().numpy(), inp.q.shape,
                              a_log=None if a_log is None else a_log.cpu().numpy())
    return inp, gate, a_log, alpha


def _to(x, d):
    return None if x is None else x.to(d)


def _accept(B, N, seed):
    """Seeded accepted-prefix lengths in [0, N], with 0 and N present."""
    g = torch.Generator().manual_seed(seed)
    n = torch.randint(0, N + 1, (B,), generator=g, dtype=torch.int32)
    n[0] = N
    if B > 1:
        n[1] = 0
    return n


def _oracle_commit(inp, alpha, n_acc):
    """Final states after each session's accepted prefix (packed oracle run)."""
    B = inp.q.shape[0]
    lens = [int(x) for x in n_acc]
    sel = lambda x: torch.cat([x[b, :lens[b]] for b in range(B)])[None]  # noqa: E731
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    a = torch.as_tensor(alpha)
    _, s = oracle.recurrent(sel(inp.q.cpu()), sel(inp.k.cpu()), sel(inp.v.cpu()), sel(a),
                            sel(inp.beta.cpu()), cu_seqlens=cu, initial_state=inp.state.cpu())
    return s


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("qkv", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N", [5, 8, 12])
def test_verify_and_commit_against_oracle(Dk, Dv, qkv, N):
    """Five drafts step the tokens; eight take the chunk form for verify (its
    stacked form of up to eight drafts), twelve for both calls."""
    d = dev()
    B, H = 3, 4
    inp, gate, a_log, alpha = _case(B, N, H, Dk, Dv, seed=900 + Dk + Dv + N, qkv=qkv)
    tol = TOL_F32 if qkv == torch.float32 else TOL_BF16
    state = inp.state.to(d)
    s0 = state.clone()
    o = kda.decode_verify(inp.q.to(d), inp.k.to(d), inp.v.to(d), gate.to(d), inp.beta.to(d),
                          state)
    torch.cuda.synchronize()
    assert torch.equal(state, s0)  # verify leaves the state alone
    o_ref, _ = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta, initial_state=inp.state)
    close(o, o_ref, tol, "tokens")
    n_acc = _accept(B, N, seed=901)
    kda.decode_commit(inp.k.to(d), inp.v.to(d), gate.to(d), inp.beta.to(d), n_acc.to(d), state)
    torch.cuda.synchronize()
    s_ref = _oracle_commit(inp, alpha, n_acc)
    close(state, s_ref, tol, "state")
    assert torch.equal(state[1], s0[1])  # nothing accepted: untouched


@pytest.mark.parametrize("kind", ["alpha", "log", "bounded", "scalar", "none"])
@pytest.mark.parametrize("N", [3, 9, 16])
def test_spec_round_against_single_steps(kind, N):
    """Verify outputs against the outputs of N decode steps, and commit of m
    tokens against the state of m decode steps: bitwise for three drafts (the
    same token loop), within fp32 rounding (1e-5 per bucket) for 9 (verify in
    the chunk form) and 16 (both calls in the chunk form)."""
    d = dev()
    B, H, D = 2, 3, 128
    inp, gate, a_log, _ = _case(B, N, H, D, D, seed=910 + N, kind=kind)
    q, k, v, beta = (x.to(d) for x in (inp.q, inp.k, inp.v, inp.beta))
    g, al = _to(gate, d), _to(a_log, d)
    o = kda.decode_verify(q, k, v, g, beta, inp.state.to(d), gate=kind, a_log=al)
    st = inp.state.to(d)
    o_steps, states = [], []
    for t in range(N):
        gt = None if g is None else g[:, t].contiguous()
        o_steps.append(kda.decode_step(q[:, t].contiguous(), k[:, t].contiguous(),
                                       v[:, t].contiguous(), gt, beta[:, t].contiguous(), st,
                                       gate=kind, a_log=al))
        states.append(st.clone())
    torch.cuda.synchronize()
    o_steps = torch.stack(o_steps, dim=1)
    if N == 3:
        assert torch.equal(o, o_steps)
    else:
        close(o, o_steps, TOL_F32, "steps")
    for m in sorted({1, min(4, N), N}):
        sc = inp.state.to(d)
        kda.decode_commit(k, v, g, beta, torch.full((B,), m, dtype=torch.int32, device=d), sc,
                          gate=kind, a_log=al)
        torch.cuda.synchronize()
        if N == 3:
            assert torch.equal(sc, states[m - 1]), m
        else:
            close(sc, states[m - 1], TOL_F32, "state")


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_spec_round_many_tiles(Dk, Dv):
    """768 (session, head) tiles of twelve drafts in the chunk form (several
    workgroups per compute unit, in several rounds): verify and commit of seeded
    prefixes against the oracle."""
    d = dev()
    B, N, H = 16, 12, 48
    inp, gate, a_log, alpha = _case(B, N, H, Dk, Dv, seed=960 + Dk + Dv, kind="log")
    state = inp.state.to(d)
    s0 = state.clone()
    o = kda.decode_verify(inp.q.to(d), inp.k.to(d), inp.v.to(d), gate.to(d), inp.beta.to(d),
                          state, gate="log")
    torch.cuda.synchronize()
    assert torch.equal(state, s0)
    o_ref, _ = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta, initial_state=inp.state)
    close(o, o_ref, TOL_BF16, "tokens")
    n_acc = _accept(B, N, seed=961)
    kda.decode_commit(inp.k.to(d), inp.v.to(d), gate.to(d), inp.beta.to(d), n_acc.to(d), state,
                      gate="log")
    torch.cuda.synchronize()
    close(state, _oracle_commit(inp, alpha, n_acc), TOL_BF16, "state")
    assert torch.equal(state[1], s0[1])


@pytest.mark.parametrize("N", [8, 12, 16])
def test_spec_round_fast_decay(N):
    """-log alpha ~ N(6, 0.5^2) per token and channel: over 16 drafts the decay
    leaves fp32's range, so the chunk form's decay ratios come from running
    products (the factored form would divide by it); over 8 and 12 the factored
    form divides by decays down to about e^-72.  Against the oracle and against
    single steps."""
    d = dev()
    B, H, D = 3, 2, 128
    inp, _, _, _ = _case(B, N, H, D, D, seed=940 + N)
    z = torch.randn(inp.alpha.shape, generator=torch.Generator().manual_seed(941 + N))
    alpha = torch.exp(-(6.0 + 0.5 * z)).float()
    q, k, v, beta, a = (x.to(d) for x in (inp.q, inp.k, inp.v, inp.beta, alpha))
    st = inp.state.to(d)
    o = kda.decode_verify(q, k, v, a, beta, st)
    o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta, initial_state=inp.state)
    st_steps = inp.state.to(d)
    o_steps = torch.stack([kda.decode_step(q[:, t].contiguous(), k[:, t].contiguous(),
                                           v[:, t].contiguous(), a[:, t].contiguous(),
                                           beta[:, t].contiguous(), st_steps)
                           for t in range(N)], dim=1)
    kda.decode_commit(k, v, a, beta, torch.full((B,), N, dtype=torch.int32, device=d), st)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(st).all()
    close(o, o_ref, TOL_BF16, "tokens")
    close(st, s_ref, TOL_BF16, "state")
    close(o, o_steps, TOL_F32, "steps")
    close(st, st_steps, TOL_F32, "state")


def test_draft_lengths_and_clamping():
    """N = 1 and N = 16 (the maximum); n_accept outside [0, N] is clamped."""
    d = dev()
    for N in (1, 16):
        inp, gate, _, alpha = _case(2, N, 2, 128, 128, seed=920 + N)
        state = inp.state.to(d)
        o = kda.decode_verify(inp.q.to(d), inp.k.to(d), inp.v.to(d), gate.to(d),
                              inp.beta.to(d), state, out_dtype=torch.bfloat16)
        o_ref, s_ref = oracle.recurrent(inp.q, inp.k, inp.v, alpha, inp.beta,
                                        initial_state=inp.state)
        torch.cuda.synchronize()
        close(o.float(), o_ref, TOL_BF16_OUT, "tokens")
        n_acc = torch.tensor([N + 5, -3], dtype=torch.int32, device=d)
        kda.decode_commit(inp.k.to(d), inp.v.to(d), gate.to(d), inp.beta.to(d), n_acc, state)
        torch.cuda.synchronize()
        close(state[0:1], s_ref[0:1], TOL_BF16, "state")
        assert torch.equal(state[1].cpu(), inp.state[1])
    with pytest.raises(kda.KdaError):
        inp, gate, _, _ = _case(1, 17, 1, 128, 128, seed=929)
        kda.decode_verify(inp.q.to(d), inp.k.to(d), inp.v.to(d), gate.to(d), inp.beta.to(d),
                          inp.state.to(d))


def test_spec_decode_b64_n8_bounded_gate():
    """Serving shape: 64 sessions x 96 heads x 128 x 128 fp32 state, 8 draft
    tokens each with K3's bounded gate; seeded acceptance."""
    d = dev()
    B, N, H, D = 64, 8, 96, 128
    inp, gate, a_log, alpha = _case(B, N, H, D, D, seed=1006, kind="bounded", device=d)
    state = inp.state.clone()
    o = kda.decode_verify(inp.q, inp.k, inp.v, gate, inp.beta, state, gate="bounded",
                          a_log=a_log)
    n_acc = _accept(B, N, seed=1007).to(d)
    kda.decode_commit(inp.k, inp.v, gate, inp.beta, n_acc, state, gate="bounded", a_log=a_log)
    torch.cuda.synchronize()
    cpu = synth.KdaInputs(inp.q.cpu(), inp.k.cpu(), inp.v.cpu(), None, inp.beta.cpu(),
                          inp.state.cpu())
    o_ref, _ = oracle.recurrent(cpu.q, cpu.k, cpu.v, alpha, cpu.beta, initial_state=cpu.state)
    close(o, o_ref, TOL_BF16, "tokens")
    s_ref = _oracle_commit(cpu, alpha, n_acc.cpu())
    close(state, s_ref, TOL_BF16, "state")
