"""Speculative decoding on the GPU: verify (N draft tokens stepped from the state,
which stays untouched) and commit (the accepted prefix replayed into the state),
against the fp64 oracle and bitwise against N single decode steps."""
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
def test_verify_and_commit_against_oracle(Dk, Dv, qkv):
    d = dev()
    B, N, H = 3, 7, 4
    inp, gate, a_log, alpha = _case(B, N, H, Dk, Dv, seed=900 + Dk + Dv, qkv=qkv)
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
def test_spec_round_equals_single_steps_bitwise(kind):
    """Verify outputs are bitwise the outputs of N decode steps, and commit of m
    tokens leaves bitwise the state of m decode steps."""
    d = dev()
    B, N, H, D = 2, 9, 3, 128
    inp, gate, a_log, _ = _case(B, N, H, D, D, seed=910, kind=kind)
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
    assert torch.equal(o, torch.stack(o_steps, dim=1))
    for m in (1, 4, N):
        sc = inp.state.to(d)
        kda.decode_commit(k, v, g, beta, torch.full((B,), m, dtype=torch.int32, device=d), sc,
                          gate=kind, a_log=al)
        torch.cuda.synchronize()
        assert torch.equal(sc, states[m - 1]), m


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
