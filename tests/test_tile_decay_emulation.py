"""CPU emulation of how the chunked kernels factor the decay inside a 64-token
chunk, against the fp64 token recurrence (the oracle).

The chunk form needs, for tokens j <= r of a chunk, the decay ratio
Gamma_r / Gamma_j = alpha_{j+1} ... alpha_r per key channel ("Kimi Delta
Attention 完全拆解", section "chunk 内并行、chunk 间递推"; "Kimi K3 的 KDA" section 5).
The kernels cut the chunk into 16-token tiles.  A pair in different tiles is
factored as (q_r P_r) . (k_j S_j E_between) with P the running product from
the start of r's tile, S the product after j to the end of j's tile and E the
whole-tile products between: every factor is at most 1.  A pair in the same
tile is factored as (q_r P_r) . (k_j / P_j), whose second factor overflows fp32
once a tile's decay product drops below about 1e-38 -- the unbounded gate
allows that ("Kimi K3 的 KDA" section 6; "Kimi K3模型架构详解" section 3.4 give the
lower bound that prevents it for K3's gate).  Tiles whose whole-tile product
falls below 2^-116 in any channel therefore take running products restarted
after j instead.  This emulation computes the factors in fp32, as the kernels
do, and everything else in fp64, and shows (1) the factored diagonal tile
breaks down on fast decay, (2) the exact path reproduces the recurrence there
and (3) on ordinary decay both paths agree with it."""
import numpy as np

import oracle

TILE_MIN = np.float32(2.0 ** -116)


def _chunk_factors(a, exact_tiles):
    """Decay ratios R[r, j, c] = prod_{s=j+1..r} a[s, c] for j <= r of one chunk
    ([C, Dk] decays), through the kernels' factors in fp32.  exact_tiles: None
    (decide per tile by the 2^-116 rule), True or False (force)."""
    a = a.astype(np.float32)
    C, Dk = a.shape
    nt = C // 16
    P = np.empty_like(a)          # running product from the tile start
    S = np.empty_like(a)          # product after the token to the tile end
    E = np.empty((nt, Dk), dtype=np.float32)
    for t in range(nt):
        blk = a[16 * t:16 * t + 16]
        run = np.ones(Dk, dtype=np.float32)
        for i in range(16):
            run = run * blk[i]
            P[16 * t + i] = run
        E[t] = run
        run = np.ones(Dk, dtype=np.float32)
        for i in range(15, -1, -1):
            S[16 * t + i] = run
            run = run * blk[i]
    R = np.zeros((C, C, Dk), dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        for m in range(nt):
            flagged = bool(np.any(E[m] < TILE_MIN)) if exact_tiles is None else exact_tiles
            for n in range(m + 1):
                for r in range(16 * m, 16 * m + 16):
                    for j in range(16 * n, 16 * n + 16):
                        if j > r:
                            continue
                        if n < m:
                            between = np.ones(Dk, dtype=np.float32)
                            for i in range(n + 1, m):
                                between = between * E[i]
                            R[r, j] = P[r] * (S[j] * between)
                        elif flagged:
                            run = np.ones(Dk, dtype=np.float32)
                            for s in range(j + 1, r + 1):
                                run = run * a[s]
                            R[r, j] = run
                        else:
                            R[r, j] = P[r] * (np.float32(1.0) / P[j])
    return R


def _chunked(q, k, v, a, b, S0, exact_tiles=None):
    """The chunk form of one (sequence, head) with the emulated factors (T a
    multiple of 64): returns (o, S)."""
    T, Dk = k.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, 64):
        sl = slice(c0, c0 + 64)
        qc, kc, vc, ac, bc = q[sl], k[sl], v[sl], a[sl], b[sl]
        R = _chunk_factors(ac, exact_tiles)
        G = np.cumprod(ac.astype(np.float64), axis=0)   # Gamma_r (for Gamma*Q, Gamma*K)
        A = np.einsum("rc,jc,rjc->rj", kc, kc, R) * bc[:, None]
        A = np.tril(A, -1)
        Mqk = np.tril(np.einsum("rc,jc,rjc->rj", qc, kc, R))
        Tm = np.linalg.inv(np.eye(64) + A)
        W = Tm @ (bc[:, None] * (G * kc))
        U = Tm @ (bc[:, None] * vc)
        P = U - W @ S
        o[sl] = (G * qc) @ S + Mqk @ P
        gC = G[-1]
        # Gamma_C / Gamma_j for every token j: the product after j to the chunk end
        Ktil = np.stack([np.prod(ac[j + 1:].astype(np.float64), axis=0) for j in range(64)]) * kc
        S = gC[:, None] * S + Ktil.T @ P
    return o, S


def _inputs(rng, T, Dk, Dv, neg_log_alpha):
    q = rng.standard_normal((T, Dk))
    k = rng.standard_normal((T, Dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, Dv))
    a = np.exp(-neg_log_alpha(rng, (T, Dk))).astype(np.float32).astype(np.float64)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = 0.02 * rng.standard_normal((Dk, Dv))
    return q, k, v, a, b, S0


def _ref(q, k, v, a, b, S0):
    o, S = oracle.recurrent(q[None, :, None], k[None, :, None], v[None, :, None],
                            a[None, :, None], b[None, :, None], initial_state=S0[None, None])
    return o[0, :, 0], S[0, 0]


def test_fast_decay_breaks_the_factored_tile_and_the_exact_path_holds():
    """-log alpha ~ 6 per token: a 16-token tile decays by ~e^-96 < 2^-116."""
    rng = np.random.default_rng(5)
    q, k, v, a, b, S0 = _inputs(rng, 128, 16, 8, lambda r, s: 6.0 + 0.5 * r.standard_normal(s))
    o_ref, S_ref = _ref(q, k, v, a, b, S0)
    with np.errstate(all="ignore"):
        o_f, S_f = _chunked(q, k, v, a, b, S0, exact_tiles=False)
    assert not (np.all(np.isfinite(o_f)) and np.all(np.isfinite(S_f)))
    o_e, S_e = _chunked(q, k, v, a, b, S0)  # the 2^-116 rule flags these tiles
    assert oracle.rel_l2(o_e, o_ref) < 1e-5 and oracle.rel_l2(S_e, S_ref) < 1e-5


def test_mixed_channels_one_fast_channel_flags_the_tile():
    """Ordinary decay everywhere but one channel that decays by e^-40 a token:
    the tile is flagged and the result still matches."""
    rng = np.random.default_rng(6)

    def nla(r, s):
        x = np.log1p(np.exp(r.standard_normal(s) + 1.0))
        x[:, 3] = 40.0
        return x
    q, k, v, a, b, S0 = _inputs(rng, 128, 16, 8, nla)
    o_ref, S_ref = _ref(q, k, v, a, b, S0)
    o_e, S_e = _chunked(q, k, v, a, b, S0)
    assert oracle.rel_l2(o_e, o_ref) < 1e-5 and oracle.rel_l2(S_e, S_ref) < 1e-5


def test_ordinary_decay_both_paths_agree_with_the_recurrence():
    """The workloads' gate exp(-softplus(N(0,1) + 1)): no tile is flagged, and
    forcing the exact path changes nothing beyond fp32 rounding."""
    rng = np.random.default_rng(7)
    q, k, v, a, b, S0 = _inputs(rng, 128, 16, 8,
                                lambda r, s: np.log1p(np.exp(r.standard_normal(s) + 1.0)))
    o_ref, S_ref = _ref(q, k, v, a, b, S0)
    o_f, S_f = _chunked(q, k, v, a, b, S0, exact_tiles=False)
    o_e, S_e = _chunked(q, k, v, a, b, S0, exact_tiles=True)
    for o, S in ((o_f, S_f), (o_e, S_e)):
        assert oracle.rel_l2(o, o_ref) < 1e-5 and oracle.rel_l2(S, S_ref) < 1e-5
