"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Each test names the passage it follows.  None of them re-types the oracle's own
loop: they use brute force, closed forms, invariants, finite differences or an
independent formulation (explicit transition matrices, the chunk form).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, B, T, H, Dk, Dv, unit_k=True, alpha_lo=0.3, beta=None):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    a = rng.uniform(alpha_lo, 1.0, (B, T, H, Dk))
    b = rng.uniform(0.05, 0.95, (B, T, H)) if beta is None else np.full((B, T, H), beta)
    return q, k, v, a, b


def test_linear_attention_bruteforce():
    """alpha = 1, no erase, beta = 1 is linear attention: o_t = sum_{i<=t} (q_t.k_i) v_i.
    "Kimi K3 的 KDA" section 2; "Kimi Delta Attention 完全拆解", section
    "线性注意力是一张矩阵形式的关联表"."""
    rng = np.random.default_rng(1)
    B, T, H, Dk, Dv = 2, 48, 2, 8, 6
    q, k, v, _, _ = _rand(rng, B, T, H, Dk, Dv, unit_k=False)
    a = np.ones((B, T, H, Dk))
    b = np.ones((B, T, H))
    o, S = oracle.recurrent(q, k, v, a, b, mode="erase_off")
    ref = np.zeros_like(o)
    for bb in range(B):
        for h in range(H):
            for t in range(T):
                for i in range(t + 1):
                    ref[bb, t, h] += np.dot(q[bb, t, h], k[bb, i, h]) * v[bb, i, h]
    assert np.max(np.abs(o - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))
    # state is the sum of outer products k_i v_i^T
    Sref = np.einsum("bthk,bthv->bhkv", k, v)
    assert np.max(np.abs(S - Sref)) < 1e-12 * np.max(np.abs(Sref))


def test_exact_overwrite_unit_key():
    """Unit-norm k, beta = 1, alpha = 1: after each step S_t^T k_t = v_t exactly
    ("从线性注意力到 KDA", section "一步在线学习": the regression minimum;
    "Kimi Delta Attention 完全拆解", section "Delta Rule 先计算写入误差").
    Read-out with q_t = k_t returns S_t^T k_t, so o_t must equal v_t."""
    rng = np.random.default_rng(2)
    B, T, H, Dk, Dv = 1, 40, 3, 16, 12
    _, k, v, _, _ = _rand(rng, B, T, H, Dk, Dv)
    s0 = rng.standard_normal((B, H, Dk, Dv))
    o, S = oracle.recurrent(k, k, v, np.ones_like(k), np.ones((B, T, H)), initial_state=s0)
    assert np.max(np.abs(o - v)) < 1e-13 * 10
    last = np.einsum("bhkv,bhk->bhv", S, k[:, -1])
    assert np.max(np.abs(last - v[:, -1])) < 1e-12


def test_beta_zero_pure_decay_closed_form():
    """beta = 0 only forgets: S_t = Diag(prod_{r<=t} alpha_r) S_0 and
    o_t = S_0^T (Gamma_t * q_t) ("Kimi Delta Attention 完全拆解", section "KDA 的核心",
    degenerate cases)."""
    rng = np.random.default_rng(3)
    B, T, H, Dk, Dv = 2, 30, 2, 8, 5
    q, k, v, a, _ = _rand(rng, B, T, H, Dk, Dv, alpha_lo=0.8)
    s0 = rng.standard_normal((B, H, Dk, Dv))
    o, S = oracle.recurrent(q, k, v, a, np.zeros((B, T, H)), initial_state=s0)
    gamma = np.cumprod(a, axis=1)  # [B,T,H,Dk]
    Sref = gamma[:, -1, :, :, None] * s0
    oref = np.einsum("bhkv,bthk->bthv", s0, gamma * q)
    assert np.max(np.abs(S - Sref)) < 1e-13
    assert np.max(np.abs(o - oref)) < 1e-13


def test_two_token_erase_free_expansion():
    """Erase-free, scalar alpha, two tokens: S_2 = a2 a1 S_in + a2 k1 v1^T + k2 v2^T
    ("Kimi K3 的 KDA", section 5, the two-token example)."""
    rng = np.random.default_rng(4)
    Dk, Dv = 5, 4
    k = rng.standard_normal((1, 2, 1, Dk))
    v = rng.standard_normal((1, 2, 1, Dv))
    q = rng.standard_normal((1, 2, 1, Dk))
    a1, a2 = 0.7, 0.4
    a = np.stack([np.full(Dk, a1), np.full(Dk, a2)])[None, :, None, :]
    s_in = rng.standard_normal((1, 1, Dk, Dv))
    _, S = oracle.recurrent(q, k, v, a, np.ones((1, 2, 1)), initial_state=s_in, mode="erase_off")
    ref = a2 * a1 * s_in[0, 0] + a2 * np.outer(k[0, 0, 0], v[0, 0, 0]) + np.outer(k[0, 1, 0], v[0, 1, 0])
    assert np.max(np.abs(S[0, 0] - ref)) < 1e-14


def test_one_gradient_step_on_decayed_state():
    """S_t = Sbar - beta grad L(Sbar), L(S) = 1/2 ||S^T k - v||^2, Sbar = Diag(alpha) S_{t-1}
    ("Kimi Delta Attention 完全拆解", section "Delta Rule"; "从线性注意力到 KDA", section
    "一步在线学习", decay before erase).  The gradient is taken by central finite
    differences, which are exact up to rounding for a quadratic loss."""
    rng = np.random.default_rng(5)
    Dk, Dv = 6, 4
    s0 = rng.standard_normal((1, 1, Dk, Dv))
    q, k, v, a, b = _rand(rng, 1, 1, 1, Dk, Dv)
    sbar = a[0, 0, 0][:, None] * s0[0, 0]
    kk, vv = k[0, 0, 0], v[0, 0, 0]

    def loss(S):
        r = S.T @ kk - vv
        return 0.5 * float(r @ r)

    grad = np.zeros_like(sbar)
    h = 1e-3
    for i in range(Dk):
        for j in range(Dv):
            E = np.zeros_like(sbar)
            E[i, j] = h
            grad[i, j] = (loss(sbar + E) - loss(sbar - E)) / (2 * h)
    ref = sbar - b[0, 0, 0] * grad
    o, S = oracle.recurrent(q, k, v, a, b, initial_state=s0)
    assert np.max(np.abs(S[0, 0] - ref)) < 1e-9
    assert np.max(np.abs(o[0, 0, 0] - ref.T @ q[0, 0, 0])) < 1e-9


def test_matches_explicit_dplr_transition():
    """The loop equals S_t = (Diag(alpha) - (beta k)(k*alpha)^T) S_{t-1} + beta k v^T with
    explicit matrices ("从线性注意力到 KDA", section "公式 (1) 的图解", DPLR form;
    "Kimi Delta Attention 完全拆解", section on DPLR)."""
    rng = np.random.default_rng(6)
    B, T, H, Dk, Dv = 2, 37, 2, 12, 10
    q, k, v, a, b = _rand(rng, B, T, H, Dk, Dv)
    s0 = rng.standard_normal((B, H, Dk, Dv))
    o1, S1 = oracle.recurrent(q, k, v, a, b, initial_state=s0)
    o2, S2 = oracle.recurrent_matrix(q, k, v, a, b, initial_state=s0)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(S1 - S2)) < 1e-12
    # and the DPLR matrix is the product (I - beta k k^T) Diag(alpha)
    kk, aa, bb = k[0, 0, 0], a[0, 0, 0], b[0, 0, 0]
    M1 = (np.eye(Dk) - bb * np.outer(kk, kk)) @ np.diag(aa)
    M2 = np.diag(aa) - np.outer(bb * kk, kk * aa)
    assert np.max(np.abs(M1 - M2)) < 1e-15


def test_degenerate_gdn_and_deltanet():
    """Equal channels give the scalar-gate GDN form alpha (I - beta k k^T) S + beta k v^T;
    alpha = 1 gives DeltaNet S - beta k (S^T k - v)^T ("Kimi Delta Attention 完全拆解",
    sections "Gated DeltaNet 仍只有一个遗忘旋钮" and "Delta Rule")."""
    rng = np.random.default_rng(7)
    B, T, H, Dk, Dv = 1, 20, 1, 8, 6
    q, k, v, _, b = _rand(rng, B, T, H, Dk, Dv)
    s0 = rng.standard_normal((B, H, Dk, Dv))
    sc = rng.uniform(0.5, 1.0, (B, T, H))
    a = np.repeat(sc[..., None], Dk, axis=-1)
    _, S = oracle.recurrent(q, k, v, a, b, initial_state=s0)
    Sg = s0[0, 0].copy()
    for t in range(T):
        kt = k[0, t, 0]
        Sg = sc[0, t, 0] * (np.eye(Dk) - b[0, t, 0] * np.outer(kt, kt)) @ Sg \
            + b[0, t, 0] * np.outer(kt, v[0, t, 0])
    assert np.max(np.abs(S[0, 0] - Sg)) < 1e-12
    _, S = oracle.recurrent(q, k, v, np.ones_like(q), b, initial_state=s0)
    Sd = s0[0, 0].copy()
    for t in range(T):
        kt = k[0, t, 0]
        Sd = Sd - b[0, t, 0] * np.outer(kt, Sd.T @ kt - v[0, t, 0])
    assert np.max(np.abs(S[0, 0] - Sd)) < 1e-12


def _chunk_form(q, k, v, a, b, s0, C):
    """fp64 chunk form of the recurrence, written from its derivation: inside a chunk
    with entry state S, G = cumsum(log alpha); A_rj = beta_r sum_c k_rc k_jc e^{G_rc-G_jc}
    (j < r); T = (I + A)^-1; W = T Diag(beta)(e^G * K); U = T Diag(beta) V; P = U - W S;
    O = (e^G * Q) S + tril_incl(Mqk) P; S' = Diag(e^{G_C}) S + (e^{G_C - G} * K)^T P.
    ("Kimi Delta Attention 完全拆解", section "chunk 内并行、chunk 间递推";
    "Kimi K3 的 KDA" section 5)."""
    T_, Dk = q.shape
    S = s0.copy()
    o = np.zeros((T_, v.shape[1]))
    for c0 in range(0, T_, C):
        Q, K, V, Al, Bt = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C], a[c0:c0 + C], b[c0:c0 + C]
        n = Q.shape[0]
        G = np.cumsum(np.log(Al), axis=0)
        D = np.exp(G[:, None, :] - G[None, :, :])           # [r, j, c] = e^{G_rc - G_jc}
        A = Bt[:, None] * np.einsum("rc,jc,rjc->rj", K, K, D)
        A = np.tril(A, -1)
        Mqk = np.tril(np.einsum("rc,jc,rjc->rj", Q, K, D))
        Tm = np.linalg.inv(np.eye(n) + A)
        W = Tm @ (Bt[:, None] * np.exp(G) * K)
        U = Tm @ (Bt[:, None] * V)
        P = U - W @ S
        o[c0:c0 + n] = (np.exp(G) * Q) @ S + Mqk @ P
        Kt = np.exp(G[-1][None, :] - G) * K
        S = np.exp(G[-1])[:, None] * S + Kt.T @ P
    return o, S


def test_chunk_form_matches_recurrence():
    """The chunk form (with a ragged last chunk) reproduces the token loop in fp64."""
    rng = np.random.default_rng(8)
    B, T, H, Dk, Dv = 1, 83, 2, 16, 12
    q, k, v, a, b = _rand(rng, B, T, H, Dk, Dv, alpha_lo=0.5)
    s0 = rng.standard_normal((B, H, Dk, Dv))
    o, S = oracle.recurrent(q, k, v, a, b, initial_state=s0)
    for h in range(H):
        oc, Sc = _chunk_form(q[0, :, h], k[0, :, h], v[0, :, h], a[0, :, h], b[0, :, h],
                             s0[0, h], C=16)
        assert np.max(np.abs(oc - o[0, :, h])) < 1e-11
        assert np.max(np.abs(Sc - S[0, h])) < 1e-11


def test_decay_then_erase_order_matters():
    """Erase-then-decay is a different operator; the implemented order is decay first
    ("从线性注意力到 KDA", section "术语坑", last item; "Kimi Delta Attention 完全拆解",
    section "KDA 的核心": the order cannot be swapped)."""
    rng = np.random.default_rng(9)
    q, k, v, a, b = _rand(rng, 1, 64, 2, 16, 16, alpha_lo=0.2)
    o1, S1 = oracle.recurrent(q, k, v, a, b)
    o2, S2 = oracle.recurrent(q, k, v, a, b, mode="erase_then_decay")
    assert oracle.rel_l2(o2, o1) > 1e-3
    assert oracle.rel_l2(S2, S1) > 1e-3


def test_state_norm_bound():
    """For unit k and beta in [0, 1], I - beta k k^T has eigenvalues in [1 - beta, 1]
    ("从线性注意力到 KDA", section "参数化", L2 normalisation), and Diag(alpha) with
    alpha <= 1 does not expand, so ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t|| and, with
    v = 0, ||S_t||_F never grows.  Checked step by step through the state hand-off."""
    rng = np.random.default_rng(10)
    T, Dk, Dv = 50, 16, 8
    q, k, v, a, b = _rand(rng, 1, T, 1, Dk, Dv, alpha_lo=0.5)
    for vv in (v, np.zeros_like(v)):
        S = rng.standard_normal((1, 1, Dk, Dv))
        for t in range(T):
            _, S2 = oracle.recurrent(q[:, t:t + 1], k[:, t:t + 1], vv[:, t:t + 1],
                                     a[:, t:t + 1], b[:, t:t + 1], initial_state=S)
            n0, n1 = np.linalg.norm(S), np.linalg.norm(S2)
            assert n1 <= n0 + b[0, t, 0] * np.linalg.norm(vv[0, t, 0]) + 1e-12
            S = S2


def test_state_norm_bound_along_a_long_run():
    """The same bound along a long run (16384 tokens, the configs' gate
    exp(-softplus(N(0,1) + 1)) and slow decay, unit k, beta = sigmoid(N(0,1))),
    checked every 64 tokens through the state hand-off: per token
    ||S_t|| <= ||S_{t-1}|| + beta_t ||v_t|| composes to ||S_end|| <= ||S_start|| +
    sum beta_t ||v_t|| over the segment, and with v = 0 the norm never grows."""
    rng = np.random.default_rng(12)
    T, H, Dk, Dv, seg = 16384, 2, 64, 64, 64
    q, k, v, _, _ = _rand(rng, 1, T, H, Dk, Dv)
    z = rng.standard_normal((1, T, H, Dk))
    for shift in (1.0, -4.0):
        a = np.exp(-(np.maximum(z + shift, 0) + np.log1p(np.exp(-np.abs(z + shift)))))
        b = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, H))))
        for vv in (v, np.zeros_like(v)):
            S = 0.02 * rng.standard_normal((1, H, Dk, Dv))
            for t0 in range(0, T, seg):
                sl = slice(t0, t0 + seg)
                _, S2 = oracle.recurrent(q[:, sl], k[:, sl], vv[:, sl], a[:, sl], b[:, sl],
                                         initial_state=S)
                for h in range(H):
                    n0, n1 = np.linalg.norm(S[0, h]), np.linalg.norm(S2[0, h])
                    grow = np.sum(b[0, sl, h] * np.linalg.norm(vv[0, sl, h], axis=-1))
                    assert n1 <= n0 + grow + 1e-12 * (1.0 + n0)
                S = S2


def test_two_segments_equal_whole():
    """Two segments with the state handed over equal the whole sequence
    ("Kimi Delta Attention 完全拆解", section "数值路径必须以 recurrent 版本为基准校验")."""
    rng = np.random.default_rng(11)
    q, k, v, a, b = _rand(rng, 1, 90, 2, 16, 12)
    s0 = rng.standard_normal((1, 2, 16, 12))
    o, S = oracle.recurrent(q, k, v, a, b, initial_state=s0)
    cut = 37
    o1, S1 = oracle.recurrent(q[:, :cut], k[:, :cut], v[:, :cut], a[:, :cut], b[:, :cut],
                              initial_state=s0)
    o2, S2 = oracle.recurrent(q[:, cut:], k[:, cut:], v[:, cut:], a[:, cut:], b[:, cut:],
                              initial_state=S1)
    assert np.max(np.abs(np.concatenate([o1, o2], axis=1) - o)) < 1e-13
    assert np.max(np.abs(S2 - S)) < 1e-13


def test_packed_batch_isolation():
    """A packed batch gives each sequence exactly its solo result (same section:
    variable-length batches must not depend on their neighbours)."""
    rng = np.random.default_rng(12)
    lens = [5, 1, 17, 0, 9]
    q, k, v, a, b = _rand(rng, 1, sum(lens), 2, 8, 8)
    s0 = rng.standard_normal((len(lens), 2, 8, 8))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = oracle.recurrent(q, k, v, a, b, cu_seqlens=cu, initial_state=s0)
    for i, L in enumerate(lens):
        sl = slice(cu[i], cu[i + 1])
        oi, Si = oracle.recurrent(q[:, sl], k[:, sl], v[:, sl], a[:, sl], b[:, sl],
                                  initial_state=s0[i:i + 1])
        assert np.array_equal(oi, o[:, sl])
        assert np.array_equal(Si, S[i:i + 1])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(13)
    q, k, v, a, b = _rand(rng, 2, 33, 3, 16, 40)
    r1 = oracle.recurrent(q, k, v, a, b, nthreads=1)
    r2 = oracle.recurrent(q, k, v, a, b, nthreads=7)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_state_size_is_t_independent_and_matches_pages():
    """69 x 96 x 128 x 128 x 2 B = 217,055,232 B, independent of T ("Kimi K3 混合线性注意力");
    32 x 128 x 128 x 2 B = 1 MiB per layer ("Kimi Delta Attention 完全拆解", section
    "缓存从 O(T) 变成 O(1)"); about 1.68M numbers per layer with the conv cache
    ("从线性注意力到 KDA", section "每层的状态有多大")."""
    g = json.load(open(os.path.join(GOLDEN, "state_size.json")))
    rng = np.random.default_rng(14)
    H, D = 96, 128
    sizes = []
    for T in (1, 3):
        q, k, v, a, b = _rand(rng, 1, T, H, D, D)
        _, S = oracle.recurrent(q, k, v, a, b)
        sizes.append(S[0].size)
    assert sizes[0] == sizes[1] == H * D * D
    k3 = g["k3_session"]
    assert k3["layers"] * sizes[0] * k3["bytes_per_value"] == k3["total_bytes"]
    h32 = g["h32_layer"]
    assert h32["heads"] * h32["dk"] * h32["dv"] * h32["bytes_per_value"] == h32["total_bytes"]
    approx = g["k3_layer_numbers_approx"]
    # matrix state plus the last 3 projected inputs of q, k and v (kernel size 4)
    n = H * D * D + 3 * 3 * H * D
    assert round(n / 1e6, 2) == approx["approx_numbers_millions"]


def test_bad_arguments_rejected():
    rng = np.random.default_rng(15)
    q, k, v, a, b = _rand(rng, 1, 4, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v[:, :3], a, b)
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v, a, b, cu_seqlens=[0, 3, 2, 4])


def test_bounded_gate_closed_forms():
    """K3's bounded gate g = g_min Sigmoid(e^{A_h} z), alpha = e^g ("Kimi K3 的 KDA"
    section 6; "Kimi K3模型架构详解" section 3.4): Sigmoid(0) = 1/2 gives
    alpha = e^{g_min/2}; the logit limits give e^{g_min} and 1; e^{A_h} rescales
    the logit of head h only; alpha stays in (e^{g_min}, 1), so a 16-token tile
    decays by at most e^{16 g_min} = e^{-80} > 1e-35 at g_min = -5."""
    H, Dk = 3, 4
    z = np.zeros((2, H, Dk))
    a = oracle.gate_alpha("bounded", z, z.shape, a_log=np.array([0.0, 1.0, -2.0]))
    assert np.allclose(a, np.exp(-2.5), rtol=0, atol=1e-15)
    a = oracle.gate_alpha("bounded", z, z.shape, a_log=np.zeros(H), g_min=-3.0)
    assert np.allclose(a, np.exp(-1.5), rtol=0, atol=1e-15)
    big = np.full((1, H, Dk), 800.0)
    assert np.allclose(oracle.gate_alpha("bounded", big, big.shape, a_log=np.zeros(H)),
                       np.exp(-5.0), rtol=1e-15, atol=0)
    assert np.all(oracle.gate_alpha("bounded", -big, big.shape, a_log=np.zeros(H)) == 1.0)
    # head 1 has scale e^{ln 2} = 2: its alpha at z equals head 0's at 2 z
    rng = np.random.default_rng(3)
    zz = rng.standard_normal((5, 2, Dk))
    a = oracle.gate_alpha("bounded", zz, zz.shape, a_log=np.array([0.0, np.log(2.0)]))
    z2 = zz.copy(); z2[:, 0] = 2.0 * zz[:, 1]
    b = oracle.gate_alpha("bounded", z2, z2.shape, a_log=np.zeros(2))
    assert np.allclose(a[:, 1], b[:, 0], rtol=1e-14, atol=0)
    # one value by hand: z = 1, A = 0: Sigmoid(1) = e / (1 + e)
    one = np.ones((1, 1, 1))
    ref = np.exp(-5.0 * np.e / (1.0 + np.e))
    assert abs(oracle.gate_alpha("bounded", one, one.shape, a_log=np.zeros(1))[0, 0, 0] - ref) \
        < 1e-16
    # range and the 16-token tile bound
    zz = rng.standard_normal((4000, 1, 8)) * 30.0
    a = oracle.gate_alpha("bounded", zz, zz.shape, a_log=np.zeros(1))
    assert np.all(a >= np.exp(-5.0)) and np.all(a <= 1.0)
    assert np.exp(-5.0) ** 16 > 1e-35


def test_log_scalar_and_none_gates():
    """The log-space gate is log alpha; the scalar gate puts one alpha on every key
    channel; no gate is alpha = 1 ("Kimi Delta Attention 完全拆解", sections "KDA 的核心"
    and "Gated DeltaNet 仍只有一个遗忘旋钮").  With a scalar gate the decay commutes
    with the erase, alpha (I - b k k^T) S = (I - b k k^T)(alpha S), so decaying
    before or after the erase gives the same result -- which fails if the per-token
    value were spread over the wrong axis or differed across channels."""
    rng = np.random.default_rng(11)
    B, T, H, Dk, Dv = 1, 24, 2, 8, 5
    a = rng.uniform(0.2, 1.0, (B, T, H, Dk))
    assert np.allclose(oracle.gate_alpha("log", np.log(a), a.shape), a, rtol=1e-15, atol=0)
    assert np.all(oracle.gate_alpha("none", None, a.shape) == 1.0)
    sc = rng.uniform(0.2, 1.0, (B, T, H))
    sa = oracle.gate_alpha("scalar", sc, a.shape)
    assert np.all(sa == sc[..., None])
    q, k, v, _, b = _rand(rng, B, T, H, Dk, Dv)
    s0 = rng.standard_normal((B, H, Dk, Dv))
    o1, S1 = oracle.recurrent(q, k, v, sa, b, initial_state=s0)
    o2, S2 = oracle.recurrent(q, k, v, sa, b, initial_state=s0, mode="erase_then_decay")
    assert np.max(np.abs(S1 - S2)) < 1e-12 and np.max(np.abs(o1 - o2)) < 1e-12
    # ... and a per-channel gate does not commute (the order the pages fix matters)
    o3, _ = oracle.recurrent(q, k, v, a, b, initial_state=s0)
    o4, _ = oracle.recurrent(q, k, v, a, b, initial_state=s0, mode="erase_then_decay")
    assert np.max(np.abs(o3 - o4)) > 1e-3
    with pytest.raises(ValueError):
        oracle.gate_alpha("scalar", sc[:, :, :1], a.shape)
    with pytest.raises(ValueError):
        oracle.gate_alpha("softplus", a, a.shape)


def test_short_conv_pins():
    """Depthwise causal convolution, kernel 4 ("从线性注意力到 KDA", the ShortConv
    bullet; "Kimi Delta Attention 完全拆解", section "一次 KDA 前向究竟发生了什么"):
    each channel against numpy's full convolution, a one-hot kernel is a shift
    (tap 3 the current token, tap 0 three tokens back, reaching into the state),
    and a sequence cut in two with the state handed over equals the whole."""
    rng = np.random.default_rng(21)
    B, T, C = 2, 11, 5
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, 4))
    y, st = oracle.short_conv(x, w)
    for b in range(B):
        for c in range(C):
            full = np.convolve(x[b, :, c], w[c, ::-1])[:T]
            assert np.allclose(y[b, :, c], full, rtol=0, atol=1e-13)
    assert np.array_equal(st, x[:, -3:])
    s0 = rng.standard_normal((B, 3, C))
    e3 = np.zeros((C, 4)); e3[:, 3] = 1.0
    assert np.array_equal(oracle.short_conv(x, e3, s0)[0], x)
    e0 = np.zeros((C, 4)); e0[:, 0] = 1.0
    y0, _ = oracle.short_conv(x, e0, s0)
    assert np.array_equal(y0[:, :3], s0) and np.array_equal(y0[:, 3:], x[:, :-3])
    ya, sa = oracle.short_conv(x[:, :4], w, s0)
    yb, sb = oracle.short_conv(x[:, 4:], w, sa)
    yw, sw = oracle.short_conv(x, w, s0)
    assert np.allclose(np.concatenate([ya, yb], axis=1), yw, rtol=0, atol=1e-14)
    assert np.array_equal(sb, sw)
    # a cut shorter than the kernel: the state carries old inputs forward
    yc, sc = oracle.short_conv(x[:, :1], w, s0)
    assert np.array_equal(sc, np.concatenate([s0[:, 1:], x[:, :1]], axis=1))


def test_silu_l2norm_rmsnorm_gate_pins():
    """Swish(x) - Swish(-x) = x and Swish(0) = 0; L2Norm gives unit rows (eps = 0)
    and ignores scale; RMSNorm of a constant row c gives sign(c) w, the gate
    Sigmoid(0) halves it, and with w = 1 and an open gate the output has RMS 1
    ("从线性注意力到 KDA", the output norm and gate section)."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((4, 9)) * 3
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-14)
    assert oracle.silu(np.zeros(1))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    n = oracle.l2norm(x, eps=0.0)
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(oracle.l2norm(7.5 * x, eps=0.0), n, rtol=0, atol=1e-14)
    assert np.all(oracle.l2norm(np.zeros((1, 4))) == 0.0)
    w = rng.uniform(0.5, 1.5, 9)
    c = np.full((2, 9), -2.5)
    big = np.full((2, 9), 50.0)
    assert np.allclose(oracle.rmsnorm_gate(c, big, w, eps=0.0), -w, rtol=0, atol=1e-14)
    assert np.allclose(oracle.rmsnorm_gate(c, np.zeros((2, 9)), w, eps=0.0), -0.5 * w,
                       rtol=0, atol=1e-14)
    y = oracle.rmsnorm_gate(x, np.full(x.shape, 60.0), np.ones(9), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=1e-14)


def test_prologue_state_layout_and_handover():
    """The prologue's state holds the last 3 inputs of q | k | v per head; a
    prefill cut in two with the state handed over equals the whole, and each
    tensor reads its own channel range of the state (a plausible slip -- q and k
    swapped, or heads interleaved -- changes the first tokens)."""
    rng = np.random.default_rng(23)
    B, T, H, Dk, Dv = 2, 7, 3, 4, 5
    xq, xk = rng.standard_normal((2, B, T, H, Dk))
    xv = rng.standard_normal((B, T, H, Dv))
    wq, wk = rng.standard_normal((2, H, Dk, 4))
    wv = rng.standard_normal((H, Dv, 4))
    s0 = rng.standard_normal((B, 3, H, 2 * Dk + Dv))
    q, k, v, s = oracle.prologue(xq, xk, xv, wq, wk, wv, s0)
    assert np.array_equal(s[:, :, :, :Dk], xq[:, -3:]) and np.array_equal(s[:, :, :, Dk:2 * Dk], xk[:, -3:])
    assert np.array_equal(s[:, :, :, 2 * Dk:], xv[:, -3:])
    q1, k1, v1, s1 = oracle.prologue(xq[:, :2], xk[:, :2], xv[:, :2], wq, wk, wv, s0)
    q2, k2, v2, s2 = oracle.prologue(xq[:, 2:], xk[:, 2:], xv[:, 2:], wq, wk, wv, s1)
    for a, b1, b2 in ((q, q1, q2), (k, k1, k2), (v, v1, v2)):
        assert np.allclose(a, np.concatenate([b1, b2], axis=1), rtol=0, atol=1e-14)
    assert np.array_equal(s, s2)
    # token 0 of head 1, channel 0 of k by hand: taps over (state k rows, x_k)
    h, c = 1, 0
    pre = (wk[h, c, 0] * s0[0, 0, h, Dk + c] + wk[h, c, 1] * s0[0, 1, h, Dk + c]
           + wk[h, c, 2] * s0[0, 2, h, Dk + c] + wk[h, c, 3] * xk[0, 0, h, c])
    row = []
    for cc in range(Dk):
        p = (wk[h, cc, 0] * s0[0, 0, h, Dk + cc] + wk[h, cc, 1] * s0[0, 1, h, Dk + cc]
             + wk[h, cc, 2] * s0[0, 2, h, Dk + cc] + wk[h, cc, 3] * xk[0, 0, h, cc])
        row.append(p / (1.0 + np.exp(-p)))
    row = np.array(row)
    assert abs(k[0, 0, h, c] - (pre / (1 + np.exp(-pre))) / np.sqrt(np.sum(row ** 2) + 1e-6)) < 1e-13


def test_affine_summary_pins():
    """The recurrence is affine in the entry state, so a segment of tokens acts as
    S -> M S + b ("Kimi K3模型架构详解" section 3.6): applied to any entry state the
    summary equals the token loop (a different formulation: the C recurrence),
    summaries compose associatively, the empty segment is (I, 0), and with
    beta = 0 the map is the pure decay Diag(prod alpha)."""
    rng = np.random.default_rng(31)
    T, Dk, Dv = 20, 6, 5
    q, k, v, a, b = _rand(rng, 1, T, 1, Dk, Dv)
    M, bb = oracle.affine_summary(k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0])
    for _ in range(3):
        s0 = rng.standard_normal((1, 1, Dk, Dv))
        _, S = oracle.recurrent(q, k, v, a, b, initial_state=s0)
        assert np.max(np.abs(M @ s0[0, 0] + bb - S[0, 0])) < 1e-12
    cut = 7
    first = oracle.affine_summary(k[0, :cut, 0], v[0, :cut, 0], a[0, :cut, 0], b[0, :cut, 0])
    second = oracle.affine_summary(k[0, cut:, 0], v[0, cut:, 0], a[0, cut:, 0], b[0, cut:, 0])
    Mc, bc = oracle.compose_summaries(first, second)
    assert np.max(np.abs(Mc - M)) < 1e-12 and np.max(np.abs(bc - bb)) < 1e-12
    M0, b0 = oracle.affine_summary(k[0, :0, 0], v[0, :0, 0], a[0, :0, 0], b[0, :0, 0])
    assert np.array_equal(M0, np.eye(Dk)) and np.array_equal(b0, np.zeros((Dk, Dv)))
    Mz, bz = oracle.affine_summary(k[0, :, 0], v[0, :, 0], a[0, :, 0], np.zeros(T))
    assert np.allclose(Mz, np.diag(np.prod(a[0, :, 0], axis=0)), rtol=0, atol=1e-15)
    assert np.all(bz == 0.0)
