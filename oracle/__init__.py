"""fp64 CPU oracle for the Kimi Delta Attention forward operator.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``kimi_delta_attention_amd``) never imports it, and this package imports
nothing from the product; they share only the seeded input arrays.

Two independent formulations live here:

* :func:`recurrent` -- the C token loop in ``kda_oracle.c`` (decay, old value,
  corrected write, read-out), fp64, parallel over (sequence, head, column block).
  Sources: "Kimi Delta Attention 完全拆解", section "一次 KDA 前向究竟发生了什么"
  (decode sequence) and section "KDA 的核心"; "Kimi K3模型架构详解" section 3.2.
* :func:`recurrent_matrix` -- a small numpy restatement that builds each step's
  explicit transition matrix in the diagonal-plus-low-rank form
  Diag(alpha) - (beta k)(k * alpha)^T ("从线性注意力到 KDA", section "公式 (1) 的图解";
  "Kimi Delta Attention 完全拆解", section "KDA 为什么比一般 DPLR 更容易做成快 Kernel")
  and applies S <- M S + beta k v^T.  It is for tiny inputs only.

Segment summaries: :func:`affine_summary` and :func:`compose_summaries`.

Around the recurrence: :func:`gate_alpha` (the decay from each gate
parametrization) and the layer's prologue and epilogue -- :func:`short_conv`,
:func:`silu`, :func:`l2norm`, :func:`prologue` (q, k, v from the projections'
outputs, with the conv state) and :func:`rmsnorm_gate` (per-head RMSNorm and
sigmoid output gate).

Parity status: pinned (see the CPU tests) by linear-attention brute force, the
exact-overwrite property, the beta = 0 closed form, the erase-free two-token
expansion, the gradient-step derivation, the state-size arithmetic, the
chunk form and two-segment composition; the gates by closed forms and the
scalar-gate commutation; the segment summaries by the recurrence itself
(applied to a state) and their composition; the prologue / epilogue by
numpy's convolution, shift
kernels, the state hand-over and closed forms.  The general random case has no
printed values on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

MODES = {"kda": 0, "erase_off": 1, "erase_then_decay": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compiles ``kda_oracle.c`` with gcc into ``libkda_oracle.so`` (in place)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.kda_oracle_forward.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P, P, P,
                                           ctypes.c_int, ctypes.c_int]
        lib.kda_oracle_forward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact upcast to a C-contiguous fp64 numpy array (torch tensors accepted)."""
    if hasattr(x, "detach"):  # torch tensor: go through fp64 on CPU (exact for bf16/fp32)
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def recurrent(q, k, v, alpha, beta, cu_seqlens=None, initial_state=None, mode: str = "kda",
              nthreads: int | None = None):
    """Token-by-token fp64 recurrence.

    Shapes follow the operator's statement: dense ``q, k, alpha`` are
    ``[B, T, H, Dk]``, ``v`` is ``[B, T, H, Dv]``, ``beta`` is ``[B, T, H]``,
    and the state is ``[B, H, Dk, Dv]``.  With ``cu_seqlens`` (``[N+1]``) the
    inputs are packed ``[1, NTOK, H, .]`` and the state is ``[N, H, Dk, Dv]``.

    Returns ``(o, final_state)`` as fp64 numpy arrays, ``o`` shaped like ``v``.
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    if q.ndim != 4:
        raise ValueError("q must be [B, T, H, Dk]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, T, H, Dv) \
            or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("packed inputs must have B == 1")
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
        if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, end at T and be non-decreasing")
    n_seq = len(cu) - 1
    s_init = None
    if initial_state is not None:
        s_init = _f64(initial_state)
        if s_init.shape != (n_seq, H, Dk, Dv):
            raise ValueError("initial_state must be [N, H, Dk, Dv]")
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    s_final = np.zeros((n_seq, H, Dk, Dv), dtype=np.float64)
    rc = _load().kda_oracle_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu), n_seq, H, Dk, Dv,
        _ptr(s_init) if s_init is not None else None, _ptr(o), _ptr(s_final),
        MODES[mode], int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed with code {rc}")
    return o, s_final


def recurrent_matrix(q, k, v, alpha, beta, initial_state=None):
    """Explicit-transition restatement for tiny dense inputs (pure numpy, fp64).

    For each (b, h) and t: M_t = Diag(alpha_t) - (beta_t k_t)(k_t * alpha_t)^T,
    S_t = M_t S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t.
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    sf = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if initial_state is None else _f64(initial_state)[b, h].copy()
            for t in range(T):
                kt, at, bt = k[b, t, h], alpha[b, t, h], beta[b, t, h]
                M = np.diag(at) - np.outer(bt * kt, kt * at)
                S = M @ S + bt * np.outer(kt, v[b, t, h])
                o[b, t, h] = S.T @ q[b, t, h]
            sf[b, h] = S
    return o, sf


def affine_summary(k, v, alpha, beta):
    """The affine map of one segment of tokens on the state, S_end = M S_start + b
    (the segment summary that lets segments of one sequence be processed in
    parallel and composed afterwards: "Kimi K3模型架构详解" section 3.6, the summaries
    (M, b) and their associative composition).

    ``k, alpha`` [T, Dk], ``v`` [T, Dv], ``beta`` [T] for one (sequence, head).
    Built from each token's explicit transition A_t = Diag(alpha_t) -
    (beta_t k_t)(k_t * alpha_t)^T: M = A_T ... A_1 and b_t = A_t b_{t-1} +
    beta_t k_t v_t^T.  Returns (M [Dk, Dk], b [Dk, Dv]) in fp64."""
    k, v, alpha, beta = (_f64(x) for x in (k, v, alpha, beta))
    T, Dk = k.shape
    M = np.eye(Dk)
    b = np.zeros((Dk, v.shape[1]))
    for t in range(T):
        A = np.diag(alpha[t]) - np.outer(beta[t] * k[t], k[t] * alpha[t])
        M = A @ M
        b = A @ b + beta[t] * np.outer(k[t], v[t])
    return M, b


def compose_summaries(first, second):
    """The summary of a segment followed by another: (M2 M1, M2 b1 + b2)."""
    M1, b1 = first
    M2, b2 = second
    return M2 @ M1, M2 @ b1 + b2


GATES = ("alpha", "log", "bounded", "scalar", "none")


def _sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function in fp64, evaluated without overflow for either sign."""
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def gate_alpha(kind: str, gate, shape, a_log=None, g_min: float = -5.0) -> np.ndarray:
    """Per-key-channel decay alpha in fp64, shape ``shape`` = [..., H, Dk], from
    one of the gate parametrizations the pages describe (the values handed to the
    GPU, upcast exactly):

    * ``alpha``   -- alpha itself, [..., H, Dk].
    * ``log``     -- g = log alpha, [..., H, Dk]; alpha = exp(g).  The FLA code
      keeps the gate in log space ("Kimi Delta Attention 完全拆解", section
      "KDA 的核心：让遗忘从一个标量细化为逐通道向量").
    * ``bounded`` -- K3's lower-bounded gate: logits z [..., H, Dk] and a per-head
      log scale A (``a_log`` [H]); g = g_min * Sigmoid(exp(A_h) z), alpha = exp(g),
      g_min = -5 on the pages ("Kimi K3 的 KDA" section 6; "Kimi K3模型架构详解"
      section 3.4).
    * ``scalar``  -- one alpha per token and head, [..., H], the same for every
      key channel: the gated DeltaNet case of a vector gate with equal
      components ("Kimi Delta Attention 完全拆解", section "KDA 的核心").
    * ``none``    -- alpha = 1: DeltaNet (same section).
    """
    shape = tuple(shape)
    if kind == "alpha":
        a = _f64(gate)
    elif kind == "log":
        a = np.exp(_f64(gate))
    elif kind == "bounded":
        z = _f64(gate)
        scale = np.exp(_f64(a_log))  # [H]
        a = np.exp(float(g_min) * _sigmoid(scale[:, None] * z))
    elif kind == "scalar":
        a = np.repeat(_f64(gate)[..., None], shape[-1], axis=-1)
    elif kind == "none":
        a = np.ones(shape, dtype=np.float64)
    else:
        raise ValueError(f"unknown gate kind {kind!r}")
    if a.shape != shape:
        raise ValueError(f"gate {kind!r} gives shape {a.shape}, expected {shape}")
    return np.ascontiguousarray(a)


# ---------------------------------------------------------------------------
# The steps on either side of the recurrence in a KDA layer ("Kimi Delta
# Attention 完全拆解", section "一次 KDA 前向究竟发生了什么", formulas for q, k, v and
# the output; "从线性注意力到 KDA", the bullet list of the layer's inputs and the
# section on the per-head output norm and gate).  The projections themselves are
# not part of the operator: their outputs are the inputs here.

def short_conv(x, w, state=None):
    """Depthwise causal convolution with kernel size 4 along the token axis.

    ``x`` [B, T, C] (C = heads x head dim, each channel on its own), ``w`` [C, 4]
    with tap 3 weighting the current token and tap j the token 3 - j before it;
    ``state`` [B, 3, C] holds the 3 inputs before the first token, oldest first
    (None: zeros).  Returns (y [B, T, C], the new state: the last 3 inputs of
    the concatenation of state and x)."""
    x = _f64(x)
    w = _f64(w)
    B, T, C = x.shape
    prev = np.zeros((B, 3, C)) if state is None else _f64(state)
    xx = np.concatenate([prev, x], axis=1)
    y = np.zeros((B, T, C))
    for j in range(4):
        y += w[:, j] * xx[:, j:j + T]
    return y, xx[:, -3:].copy()


def silu(x):
    """Swish / SiLU: x * Sigmoid(x)."""
    x = _f64(x)
    return x * _sigmoid(x)


def l2norm(x, eps: float = 1e-6):
    """x / sqrt(sum of squares over the last axis + eps)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def prologue(xq, xk, xv, wq, wk, wv, state=None, eps: float = 1e-6):
    """q, k = L2Norm(Swish(ShortConv(x_q / x_k))), v = Swish(ShortConv(x_v)).

    ``xq, xk`` [B, T, H, Dk], ``xv`` [B, T, H, Dv] (the projections' outputs);
    ``wq, wk`` [H, Dk, 4], ``wv`` [H, Dv, 4]; ``state`` [B, 3, H, 2 Dk + Dv]: the
    last 3 inputs of q | k | v before the first token (None: zeros).  Returns
    (q, k, v, new state)."""
    xq, xk, xv = _f64(xq), _f64(xk), _f64(xv)
    B, T, H, Dk = xq.shape
    Dv = xv.shape[-1]
    st = None if state is None else _f64(state).reshape(B, 3, H, 2 * Dk + Dv)
    outs, news = [], []
    for x, w, lo, D in ((xq, wq, 0, Dk), (xk, wk, Dk, Dk), (xv, wv, 2 * Dk, Dv)):
        s_in = None if st is None else st[:, :, :, lo:lo + D].reshape(B, 3, H * D)
        y, s_out = short_conv(x.reshape(B, T, H * D), _f64(w).reshape(H * D, 4), s_in)
        outs.append(silu(y).reshape(B, T, H, D))
        news.append(s_out.reshape(B, 3, H, D))
    q, k, v = outs
    return l2norm(q, eps), l2norm(k, eps), v, np.concatenate(news, axis=-1)


def rmsnorm_gate(o, g, w, eps: float = 1e-5):
    """Per-head output: RMSNorm over the head's Dv channels with weight ``w`` [Dv],
    then the sigmoid output gate, o * rsqrt(mean(o^2) + eps) * w * Sigmoid(g)."""
    o, g, w = _f64(o), _f64(g), _f64(w)
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w * _sigmoid(g)


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64."""
    x = _f64(x)
    ref = _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)
