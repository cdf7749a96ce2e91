"""The layer prefill in one call -- the prologue inside the two-pass first pass,
the recurrence, the conv state handed on, the epilogue -- against the oracle's
chain of the same steps and against the standalone calls composed."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, close, dev, rounded

pytestmark = pytest.mark.gpu

# the oracle's chain rounds q, k, v to bf16 where the prologue stores them, so
# the layer is held to the recurrence's own bar (fp32 y and o)
TOL_LAYER = TOL_BF16


def _f(x):
    return x.float().cpu()


def _inputs(B, T, H, Dk, Dv, seed, d, n_state=None):
    L = synth.make_layer(B, T, H, Dk, Dv, seed=seed, n_state=n_state, device=d)
    r = synth.make_dense(B, T, H, Dk, Dv, seed=seed + 1, state_std=0.02, device=d)
    n = B if n_state is None else n_state
    s0 = synth.make_state(n, H, Dk, Dv, seed=seed + 2, device=d)
    return L, r.alpha, r.beta, s0


def _oracle_chain(L, alpha, beta, s0, cu=None):
    """oracle prologue per sequence (each with its conv state), the recurrence
    over the packed result, RMSNorm and gate; returns (y, o, S, conv state)."""
    if cu is None:
        rq, rk, rv, rcs = oracle.prologue(_f(L.xq), _f(L.xk), _f(L.xv), L.wq, L.wk, L.wv,
                                          state=L.conv_state.cpu())
        rq, rk, rv = (rounded(x, torch.bfloat16) for x in (rq, rk, rv))
        ro, rs = oracle.recurrent(rq, rk, rv, alpha.cpu().numpy(), beta.cpu(),
                                  initial_state=s0.cpu())
    else:
        parts, states = [], []
        for i in range(len(cu) - 1):
            lo, hi = int(cu[i]), int(cu[i + 1])
            st = L.conv_state[i:i + 1].cpu()
            if hi == lo:
                states.append(st.numpy().astype(np.float64))
                continue
            q, k, v, cs = oracle.prologue(_f(L.xq[:, lo:hi]), _f(L.xk[:, lo:hi]),
                                          _f(L.xv[:, lo:hi]), L.wq, L.wk, L.wv, state=st)
            parts.append((q, k, v))
            states.append(cs)
        rq, rk, rv = (rounded(np.concatenate([p[j] for p in parts], axis=1), torch.bfloat16)
                      for j in range(3))
        rcs = np.concatenate(states, axis=0)
        ro, rs = oracle.recurrent(rq, rk, rv, alpha.cpu().numpy(), beta.cpu(), cu_seqlens=cu,
                                  initial_state=s0.cpu())
    ry = oracle.rmsnorm_gate(ro, _f(L.g), L.norm_w.cpu())
    return ry, ro, rs, rcs


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_dense_against_oracle_and_composed(Dk, Dv):
    d = dev()
    B, T, H = 2, 64 * 9 + 13, 2
    L, alpha, beta, s0 = _inputs(B, T, H, Dk, Dv, seed=1300 + Dk + Dv, d=d)
    y, o, s, cs = kda.prefill_layer(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, alpha, beta, L.g,
                                    L.norm_w, conv_state=L.conv_state, initial_state=s0)
    torch.cuda.synchronize()
    ry, ro, rs, rcs = _oracle_chain(L, alpha, beta, s0)
    close(y, ry, TOL_LAYER, "tokens")
    close(o, ro, TOL_LAYER, "tokens")
    close(s, rs, TOL_LAYER, "state")
    assert np.array_equal(cs.cpu().numpy(), rcs.astype(np.float32))  # inputs, copied exactly
    # the standalone calls composed: the same up to the L2Norm's summation order
    q, k, v, cs2 = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    o2, s2 = kda.prefill_chunked(q, k, v, alpha, beta, initial_state=s0, schedule="two_pass")
    y2 = kda.epilogue(o2, L.g, L.norm_w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(cs, cs2)
    close(y, y2, TOL_BF16, "tokens")
    close(s, s2, TOL_BF16, "state")


@pytest.mark.parametrize("n_segments", [1, 4])
def test_packed_sequences_and_windows(n_segments):
    """Empty, one-token, shorter-than-the-kernel, window-crossing and multi-chunk
    sequences packed together, each with its own conv state and state; the
    conv state of the empty one is handed through."""
    d = dev()
    lengths = [3000, 0, 2, 70, 8192 + 500, 1, 130]
    H, D = 2, 128
    tot = sum(lengths)
    L, alpha, beta, s0 = _inputs(1, tot, H, D, D, seed=1320, d=d, n_state=len(lengths))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=d)
    y, o, s, cs = kda.prefill_layer(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, alpha, beta, L.g,
                                    L.norm_w, conv_state=L.conv_state, initial_state=s0,
                                    cu_seqlens=cu, n_segments=n_segments)
    torch.cuda.synchronize()
    ry, ro, rs, rcs = _oracle_chain(L, alpha, beta, s0, cu=cu.cpu().numpy())
    close(y, ry, TOL_LAYER, "tokens", cu=cu)
    close(s, rs, TOL_LAYER, "state")
    assert np.array_equal(cs.cpu().numpy(), rcs.astype(np.float32))
    assert torch.equal(cs[1], L.conv_state[1]) and torch.equal(s[1], s0[1])


def test_bounded_gate_segments_bf16_output_no_conv_state():
    """K3's bounded gate over two windows with 6 segments, bf16 y, zero conv
    state (None) and no state out."""
    d = dev()
    B, T, H, D = 1, 9000, 3, 128
    L, _, beta, s0 = _inputs(B, T, H, D, D, seed=1340, d=d)
    z, a_log = synth.make_gate("bounded", (B, T), H, D, seed=1341, device=d)
    y, o, s, cs = kda.prefill_layer(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, z, beta, L.g, L.norm_w,
                                    initial_state=s0, n_segments=6, out_dtype=torch.bfloat16,
                                    conv_state_out=False, gate="bounded", a_log=a_log)
    torch.cuda.synchronize()
    assert cs is None and y.dtype == torch.bfloat16
    rq, rk, rv, _ = oracle.prologue(_f(L.xq), _f(L.xk), _f(L.xv), L.wq, L.wk, L.wv)
    rq, rk, rv = (rounded(x, torch.bfloat16) for x in (rq, rk, rv))
    alpha = oracle.gate_alpha("bounded", z.cpu().numpy(), (B, T, H, D), a_log=a_log.cpu().numpy())
    ro, rs = oracle.recurrent(rq, rk, rv, alpha, beta.cpu(), initial_state=s0.cpu())
    ry = oracle.rmsnorm_gate(ro, _f(L.g), L.norm_w.cpu())
    close(y.float(), ry, TOL_LAYER + 2.0 ** -8, "tokens")
    close(s, rs, TOL_LAYER, "state")


def test_empty_call_hands_states_through():
    d = dev()
    L, alpha, beta, s0 = _inputs(2, 0, 2, 128, 128, seed=1350, d=d)
    y, o, s, cs = kda.prefill_layer(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, alpha, beta, L.g,
                                    L.norm_w, conv_state=L.conv_state, initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(s, s0) and torch.equal(cs, L.conv_state)


def test_k3_8k_layer_all_heads():
    """The 8K layer (B=1, T=8192, H=96, d=128) in one call, as the bench times
    it: the oracle chain on every head and token, and the composed calls."""
    d = dev()
    B, T, H, D = 1, 8192, 96, 128
    L = synth.make_layer(B, T, H, D, D, seed=1360, device=d)
    r = synth.make_dense(B, T, H, D, D, seed=1361, state_std=0.02, device=d)
    y, o, s, cs = kda.prefill_layer(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, r.alpha, r.beta, L.g,
                                    L.norm_w, conv_state=L.conv_state, initial_state=r.state)
    q, k, v, _ = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    o2, s2 = kda.prefill_chunked(q, k, v, r.alpha, r.beta, initial_state=r.state,
                                 schedule="two_pass")
    y2 = kda.epilogue(o2, L.g, L.norm_w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    close(y, y2, TOL_BF16, "tokens")
    close(s, s2, TOL_BF16, "state")
    heads = list(range(H))
    sel = lambda x: _f(x[:, :, heads])  # noqa: E731
    st = L.conv_state[:, :, heads].cpu()
    rq, rk, rv, rcs = oracle.prologue(sel(L.xq), sel(L.xk), sel(L.xv), L.wq[heads].cpu(),
                                      L.wk[heads].cpu(), L.wv[heads].cpu(), state=st)
    rq, rk, rv = (rounded(x, torch.bfloat16) for x in (rq, rk, rv))
    ro, rs = oracle.recurrent(rq, rk, rv, r.alpha[:, :, heads].cpu().numpy(),
                              r.beta[:, :, heads].cpu(), initial_state=r.state[:, heads].cpu())
    ry = oracle.rmsnorm_gate(ro, sel(L.g), L.norm_w.cpu())
    close(y[:, :, heads], ry, TOL_LAYER, "tokens")
    close(s[:, heads], rs, TOL_LAYER, "state")
    assert np.array_equal(cs[:, :, heads].cpu().numpy(), rcs.astype(np.float32))
