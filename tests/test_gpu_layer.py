"""The layer's prologue (ShortConv + Swish + L2Norm with the conv state) and
epilogue (per-head RMSNorm and sigmoid output gate) on the GPU against the fp64
oracle, and a whole layer's prefill composed of prologue, recurrence and
epilogue against the oracle's chain of the same steps."""
import numpy as np
import pytest
import torch

import kimi_delta_attention_amd as kda
import oracle
from kimi_delta_attention_amd import synth
from tests._common import TOL_BF16, TOL_F32, close, dev, rounded

pytestmark = pytest.mark.gpu

# one rounding to nearest of the output to bf16 (8 significant bits: relative
# error <= 2^-8 per element) on top of fp32 arithmetic
TOL_ROUND = 2.0 ** -8 + 1e-5


def _f(x):
    return x.float().cpu()


def _oracle_pro(L, state, lo=None, hi=None):
    sl = slice(lo, hi)
    return oracle.prologue(_f(L.xq[:, sl]), _f(L.xk[:, sl]), _f(L.xv[:, sl]), L.wq, L.wk, L.wv,
                           state=None if state is None else state.cpu())


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_state", [True, False])
def test_prologue_dense(Dk, Dv, dtype, with_state):
    d = dev()
    L = synth.make_layer(2, 150, 3, Dk, Dv, seed=1100 + Dk + Dv, dtype=dtype, device=d)
    st = L.conv_state if with_state else None
    q, k, v, so = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=st)
    torch.cuda.synchronize()
    rq, rk, rv, rs = _oracle_pro(L, st)
    tol = TOL_ROUND if dtype == torch.bfloat16 else TOL_F32
    for a, r in ((q, rq), (k, rk), (v, rv)):
        close(a.float(), r, tol, "tokens")
    assert np.array_equal(so.cpu().numpy(), rs.astype(np.float32))  # inputs, copied exactly


def test_prologue_packed_boundaries():
    """Packed sequences that are empty, shorter than the kernel, cross the
    kernel's 64-token blocks or share one: each equals the oracle on its own, and
    each sequence's conv state (an empty one's copied through) is exact."""
    d = dev()
    lengths = [0, 1, 2, 70, 3, 0, 130, 64, 5]
    H, D = 2, 128
    tot = sum(lengths)
    L = synth.make_layer(1, tot, H, D, D, seed=1120, n_state=len(lengths), device=d)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=d)
    q, k, v, so = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state,
                               cu_seqlens=cu)
    torch.cuda.synchronize()
    c = cu.cpu().numpy()
    for i, n in enumerate(lengths):
        st_i = L.conv_state[i:i + 1]
        if n == 0:
            assert torch.equal(so[i], L.conv_state[i])
            continue
        rq, rk, rv, rs = oracle.prologue(_f(L.xq[:, c[i]:c[i + 1]]), _f(L.xk[:, c[i]:c[i + 1]]),
                                         _f(L.xv[:, c[i]:c[i + 1]]), L.wq, L.wk, L.wv,
                                         state=st_i.cpu())
        for a, r in ((q, rq), (k, rk), (v, rv)):
            close(a[:, c[i]:c[i + 1]].float(), r, TOL_ROUND, "tokens")
        assert np.array_equal(so[i:i + 1].cpu().numpy(), rs.astype(np.float32)), i


def test_prologue_handover_bitwise():
    """A prefill cut in two, the conv state handed from the first call to the
    second, gives bitwise the outputs and final state of one call."""
    d = dev()
    L = synth.make_layer(2, 200, 3, 128, 128, seed=1130, device=d)
    q, k, v, so = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    parts = []
    st = L.conv_state
    for lo, hi in ((0, 77), (77, 200)):
        sub = [x[:, lo:hi].contiguous() for x in (L.xq, L.xk, L.xv)]
        qa, ka, va, st = kda.prologue(*sub, L.wq, L.wk, L.wv, conv_state=st)
        parts.append((qa, ka, va))
    torch.cuda.synchronize()
    for j, full in enumerate((q, k, v)):
        assert torch.equal(torch.cat([p[j] for p in parts], dim=1), full)
    assert torch.equal(st, so)


@pytest.mark.parametrize("Dv", [128, 64])
@pytest.mark.parametrize("odt,gdt,ydt", [(torch.float32, torch.bfloat16, torch.bfloat16),
                                         (torch.float32, torch.float32, torch.float32),
                                         (torch.bfloat16, torch.bfloat16, torch.float32)])
def test_epilogue(Dv, odt, gdt, ydt):
    d = dev()
    L = synth.make_layer(2, 50, 3, 128, Dv, seed=1140 + Dv, dtype=gdt, device=d)
    o = (torch.randn(2, 50, 3, Dv, generator=torch.Generator(device=d).manual_seed(7),
                     device=d) * 0.3).to(odt)
    y = kda.epilogue(o, L.g, L.norm_w, out_dtype=ydt)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_gate(_f(o), _f(L.g), L.norm_w.cpu())
    close(y.float(), ref, (TOL_ROUND if ydt == torch.bfloat16 else TOL_F32), "tokens")
    if odt == ydt:  # in place over o
        o2 = o.clone()
        kda.epilogue(o2, L.g, L.norm_w, y=o2)
        torch.cuda.synchronize()
        assert torch.equal(o2, y)


@pytest.mark.parametrize("schedule", ["fused", "two_pass"])
def test_layer_prefill_composed(schedule):
    """x -> prologue -> prefill (K3's bounded gate) -> epilogue against the
    oracle's prologue -> recurrence -> RMSNorm and gate (B=1, T=300, H=4, d=128)."""
    d = dev()
    B, T, H, D = 1, 300, 4, 128
    L = synth.make_layer(B, T, H, D, D, seed=1150, device=d)
    z, a_log = synth.make_gate("bounded", (B, T), H, D, seed=1151, device=d)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=torch.Generator(device=d).manual_seed(3),
                                     device=d))
    s0 = synth.make_state(B, H, D, D, seed=1152, device=d)
    q, k, v, cso = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    o, s = kda.prefill_chunked(q, k, v, z, beta, initial_state=s0, schedule=schedule,
                               gate="bounded", a_log=a_log)
    y = kda.epilogue(o, L.g, L.norm_w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv, rcs = _oracle_pro(L, L.conv_state)
    # q, k, v enter the recurrence in the token dtype, as the prologue stores them
    rq, rk, rv = (rounded(x, torch.bfloat16) for x in (rq, rk, rv))
    alpha = oracle.gate_alpha("bounded", z.cpu().numpy(), (B, T, H, D), a_log=a_log.cpu().numpy())
    ro, rs = oracle.recurrent(rq, rk, rv, alpha, beta.cpu(), initial_state=s0.cpu())
    ry = oracle.rmsnorm_gate(ro, _f(L.g), L.norm_w.cpu())
    # q, k, v enter the recurrence rounded to bf16, as the chunked kernels take them
    close(y, ry, TOL_BF16, "tokens")
    close(s, rs, TOL_BF16, "state")
    assert np.array_equal(cso.cpu().numpy(), rcs.astype(np.float32))


def _layer_case(B, N, H, Dk, Dv, seed, kind, dtype, d):
    L = synth.make_layer(B, N, H, Dk, Dv, seed=seed, dtype=dtype, device=d)
    if kind == "alpha":
        gate, a_log = synth.make_dense(B, N, H, Dk, Dv, seed=seed, device=d).alpha, None
    else:
        gate, a_log = synth.make_gate(kind, (B, N), H, Dk, seed=seed + 1, device=d)
    beta = torch.sigmoid(torch.randn(B, N, H, generator=torch.Generator(device=d).manual_seed(seed),
                                     device=d))
    s0 = synth.make_state(B, H, Dk, Dv, seed=seed + 2, device=d)
    return L, gate, a_log, beta, s0


@pytest.mark.parametrize("kind", ["alpha", "bounded"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 128)])
def test_decode_layer_step_equals_composed(kind, dtype, Dk, Dv):
    """One fused layer step is bitwise the standalone prologue, the decode step
    (fp32 o) and the standalone epilogue, conv state and state included."""
    d = dev()
    B, H = 3, 4
    L, gate, a_log, beta, s0 = _layer_case(B, 1, H, Dk, Dv, 1200 + Dk, kind, dtype, d)
    cs, st = L.conv_state.clone(), s0.clone()
    y = kda.decode_layer("step", L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, cs, gate, beta, st, L.g,
                         L.norm_w, gate=kind, a_log=a_log, out_dtype=dtype)
    q, k, v, cso = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    st2 = s0.clone()
    o = kda.decode_step(q[:, 0], k[:, 0], v[:, 0], gate[:, 0].contiguous(), beta[:, 0].contiguous(),
                        st2, gate=kind, a_log=a_log)
    y2 = kda.epilogue(o, L.g[:, 0].contiguous(), L.norm_w, out_dtype=dtype)
    torch.cuda.synchronize()
    assert torch.equal(y[:, 0], y2) and torch.equal(st, st2) and torch.equal(cs, cso)


@pytest.mark.parametrize("kind", ["alpha", "bounded", "scalar"])
def test_decode_layer_spec_round_equals_composed(kind):
    """Fused verify bitwise the composed verify (both take the chunk form at six
    drafts), conv state and state untouched.  Fused commit of seeded prefixes:
    the state bitwise the plain commit of the prologue's k, v; the conv state
    exactly the oracle's after each prefix."""
    d = dev()
    B, N, H, D = 4, 6, 3, 128
    L, gate, a_log, beta, s0 = _layer_case(B, N, H, D, D, 1220, kind, torch.bfloat16, d)
    cs, st = L.conv_state.clone(), s0.clone()
    y = kda.decode_layer("verify", L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, cs, gate, beta, st, L.g,
                         L.norm_w, gate=kind, a_log=a_log)
    q, k, v, _ = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    o = kda.decode_verify(q, k, v, gate, beta, s0, gate=kind, a_log=a_log)
    y2 = kda.epilogue(o, L.g, L.norm_w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(cs, L.conv_state) and torch.equal(st, s0)
    n_acc = torch.tensor([N, 0, 2, 5], dtype=torch.int32, device=d)
    kda.decode_layer("commit", L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, cs, gate, beta, st,
                     n_accept=n_acc, gate=kind, a_log=a_log)
    st2 = s0.clone()
    kda.decode_commit(k, v, gate, beta, n_acc, st2, gate=kind, a_log=a_log)
    torch.cuda.synchronize()
    assert torch.equal(st, st2)
    for b, n in enumerate(n_acc.tolist()):
        if n == 0:
            assert torch.equal(cs[b], L.conv_state[b])
            continue
        *_, rs = oracle.prologue(_f(L.xq[b:b + 1, :n]), _f(L.xk[b:b + 1, :n]),
                                 _f(L.xv[b:b + 1, :n]), L.wq, L.wk, L.wv,
                                 state=L.conv_state[b:b + 1].cpu())
        assert np.array_equal(cs[b:b + 1].cpu().numpy(), rs.astype(np.float32)), b


def test_decode_layer_steps_against_oracle():
    """Seven fused layer steps from given conv and recurrent states against the
    oracle's prologue, recurrence and epilogue over the seven tokens."""
    d = dev()
    B, T, H, D = 2, 7, 4, 128
    L, gate, a_log, beta, s0 = _layer_case(B, T, H, D, D, 1240, "bounded", torch.bfloat16, d)
    cs, st = L.conv_state.clone(), s0.clone()
    ys = []
    for t in range(T):
        sl = lambda x: x[:, t:t + 1].contiguous()  # noqa: E731
        ys.append(kda.decode_layer("step", sl(L.xq), sl(L.xk), sl(L.xv), L.wq, L.wk, L.wv, cs,
                                   sl(gate), sl(beta), st, sl(L.g), L.norm_w, gate="bounded",
                                   a_log=a_log))
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=1)
    rq, rk, rv, rcs = oracle.prologue(_f(L.xq), _f(L.xk), _f(L.xv), L.wq, L.wk, L.wv,
                                      state=L.conv_state.cpu())
    rq, rk, rv = (rounded(x, torch.bfloat16) for x in (rq, rk, rv))
    alpha = oracle.gate_alpha("bounded", gate.cpu().numpy(), (B, T, H, D), a_log=a_log.cpu().numpy())
    ro, rs = oracle.recurrent(rq, rk, rv, alpha, beta.cpu(), initial_state=s0.cpu())
    ry = oracle.rmsnorm_gate(ro, _f(L.g), L.norm_w.cpu())
    close(y, ry, TOL_BF16, "tokens")
    close(st, rs, TOL_BF16, "state")
    assert np.array_equal(cs.cpu().numpy(), rcs.astype(np.float32))


def test_decode_layer_max_draft():
    """16 draft tokens (the largest LDS footprint of the fused layer): verify
    and commit bitwise the composed calls, the conv state too."""
    d = dev()
    B, N, H, D = 2, 16, 2, 128
    L, gate, a_log, beta, s0 = _layer_case(B, N, H, D, D, 1260, "alpha", torch.bfloat16, d)
    cs, st = L.conv_state.clone(), s0.clone()
    y = kda.decode_layer("verify", L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, cs, gate, beta, st, L.g,
                         L.norm_w)
    q, k, v, cso = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    y2 = kda.epilogue(kda.decode_verify(q, k, v, gate, beta, s0), L.g, L.norm_w,
                      out_dtype=torch.float32)
    n_acc = torch.full((B,), N, dtype=torch.int32, device=d)
    kda.decode_layer("commit", L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, cs, gate, beta, st,
                     n_accept=n_acc)
    st2 = s0.clone()
    kda.decode_commit(k, v, gate, beta, n_acc, st2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.equal(st, st2)
    assert torch.equal(cs, cso)


@pytest.mark.parametrize("N", [4, 7, 12])
@pytest.mark.parametrize("dtype,Dk,Dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64),
                                         (torch.bfloat16, 64, 128), (torch.float32, 128, 128)])
@pytest.mark.parametrize("decay", ["normal", "fast"])
def test_decode_layer_verify_forms(N, dtype, Dk, Dv, decay):
    """Fused verify in each form (4 drafts: the token loop; 7: the chunk form
    with K and Q stacked; 12: the chunk form) bitwise the composed calls, and
    against the oracle's prologue, recurrence and epilogue.  With -log alpha ~
    N(6, 0.5^2) the decay over the drafts leaves the factored range, so the
    chunk form's decay ratios come from running products of the prologue's k."""
    d = dev()
    B, H = 3, 2
    seed = 1280 + N + Dk + (7 if decay == "fast" else 0)
    L, gate, a_log, beta, s0 = _layer_case(B, N, H, Dk, Dv, seed, "alpha", dtype, d)
    if decay == "fast":
        z = torch.randn(gate.shape, generator=torch.Generator().manual_seed(seed))
        gate = torch.exp(-(6.0 + 0.5 * z)).float().to(d)
    cs, st = L.conv_state.clone(), s0.clone()
    y = kda.decode_layer("verify", L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, cs, gate, beta, st, L.g,
                         L.norm_w, out_dtype=torch.float32)
    q, k, v, _ = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    y2 = kda.epilogue(kda.decode_verify(q, k, v, gate, beta, s0), L.g, L.norm_w,
                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    assert torch.equal(y, y2)
    assert torch.equal(cs, L.conv_state) and torch.equal(st, s0)
    rq, rk, rv, _ = oracle.prologue(_f(L.xq), _f(L.xk), _f(L.xv), L.wq, L.wk, L.wv,
                                    state=L.conv_state.cpu())
    rq, rk, rv = (rounded(x, dtype) for x in (rq, rk, rv))
    ro, _ = oracle.recurrent(rq, rk, rv, gate.cpu().double(), beta.cpu(), initial_state=s0.cpu())
    ry = oracle.rmsnorm_gate(ro, _f(L.g), L.norm_w.cpu())
    close(y, ry, TOL_BF16, "tokens")


@pytest.mark.parametrize("N", [4, 12, 16])
@pytest.mark.parametrize("dtype,Dk,Dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64),
                                         (torch.bfloat16, 64, 128), (torch.float32, 128, 128)])
@pytest.mark.parametrize("decay", ["normal", "fast"])
def test_decode_layer_commit_forms(N, dtype, Dk, Dv, decay):
    """Fused commit in each form (4 drafts: the token loop; 12 and 16: the chunk
    form) of accepted prefixes 0, 1, 2, 3 and N (the conv state's new rows then
    come from the old rows, the tokens or both): the state bitwise the plain
    commit of the prologue's k and v and against the oracle's recurrence over
    the prefix; the conv state exactly the oracle's after the prefix.  With
    -log alpha ~ N(6, 0.5^2) the chunk form takes its running-product path."""
    d = dev()
    B, H = 5, 2
    seed = 1300 + N + Dk + (7 if decay == "fast" else 0)
    L, gate, a_log, beta, s0 = _layer_case(B, N, H, Dk, Dv, seed, "alpha", dtype, d)
    if decay == "fast":
        z = torch.randn(gate.shape, generator=torch.Generator().manual_seed(seed))
        gate = torch.exp(-(6.0 + 0.5 * z)).float().to(d)
    n_acc = torch.tensor([0, 1, 2, min(3, N), N], dtype=torch.int32, device=d)
    cs, st = L.conv_state.clone(), s0.clone()
    kda.decode_layer("commit", L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, cs, gate, beta, st,
                     n_accept=n_acc)
    _, k, v, _ = kda.prologue(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, conv_state=L.conv_state)
    st2 = s0.clone()
    kda.decode_commit(k, v, gate, beta, n_acc, st2)
    torch.cuda.synchronize()
    assert torch.isfinite(st).all()
    assert torch.equal(st, st2)
    for b, n in enumerate(n_acc.tolist()):
        if n == 0:
            assert torch.equal(cs[b], L.conv_state[b]) and torch.equal(st[b], s0[b])
            continue
        rq, rk, rv, rcs = oracle.prologue(_f(L.xq[b:b + 1, :n]), _f(L.xk[b:b + 1, :n]),
                                          _f(L.xv[b:b + 1, :n]), L.wq, L.wk, L.wv,
                                          state=L.conv_state[b:b + 1].cpu())
        assert np.array_equal(cs[b:b + 1].cpu().numpy(), rcs.astype(np.float32)), b
        rk, rv = (rounded(x, dtype) for x in (rk, rv))
        _, rs = oracle.recurrent(rounded(rq, dtype), rk, rv, gate[b:b + 1, :n].cpu().double(),
                                 beta[b:b + 1, :n].cpu(), initial_state=s0[b:b + 1].cpu())
        close(st[b:b + 1], rs, TOL_BF16, "state")
