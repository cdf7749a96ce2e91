"""Seeded synthetic inputs for the KDA forward operator.

This module only draws random numbers and shapes them into the operator's
inputs; it holds none of the operator's arithmetic.  Both the HIP path and the
CPU oracle receive exactly the arrays made here.

Distributions (the workload recipe):

* q, k  ~ N(0, 1) per element, L2-normalised per (token, head) in fp64, then
  rounded once (round-to-nearest-even) to the input dtype.  Normalised q, k are
  what the operator sees after the layer's L2Norm ("从线性注意力到 KDA", section
  "参数化"; "Kimi Delta Attention 完全拆解", section "一次 KDA 前向究竟发生了什么").
* v ~ N(0, 1), rounded to the input dtype.
* alpha = exp(-softplus(z + shift)), z ~ N(0, 1), evaluated in fp64 and stored
  fp32 -- the negative-softplus gate of Kimi Linear ("Kimi K3 的 KDA", section 6).
  shift = 0 or 1 for the standard workloads; shift = -4 gives a slow-decay
  stress input (mean alpha about 0.97); ``alpha_one=True`` gives alpha = 1.
* beta = sigmoid(N(0, 1)) in fp64, stored fp32.
* initial state ~ N(0, state_std^2) fp32 when requested.
* layer inputs (``make_layer``): the projections' outputs x_q, x_k, x_v and the
  output-gate logits g ~ N(0, 1) in the token dtype; conv taps ~ N(0, 0.5^2)
  fp32 [H, D, 4]; a conv state ~ N(0, 1) fp32 [N, 3, H, 2 Dk + Dv]; the RMSNorm
  weight ~ U(0.5, 1.5) fp32 [Dv].
* decay in another gate parametrization (``make_gate``): 'log' stores
  -softplus(z + shift) (the same decays, in log space); 'bounded' stores the
  logits z ~ N(0, 1) with a per-head log scale A ~ U(-1, 1); 'scalar' stores
  exp(-softplus(z + shift)) with one z per (token, head); 'none' stores nothing.

Token tensors are drawn in fixed blocks of ``BLOCK`` tokens, each from its own
generator seeded with (seed, block index), so a long input never needs an fp64
copy of the whole tensor and the values do not depend on the device memory
available.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

BLOCK = 8192


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _softplus64(x: torch.Tensor) -> torch.Tensor:
    return torch.clamp(x, min=0) + torch.log1p(torch.exp(-x.abs()))


@dataclass
class KdaInputs:
    q: torch.Tensor          # [B, T, H, Dk]
    k: torch.Tensor          # [B, T, H, Dk]
    v: torch.Tensor          # [B, T, H, Dv]
    alpha: torch.Tensor      # [B, T, H, Dk] fp32
    beta: torch.Tensor       # [B, T, H] fp32
    state: torch.Tensor | None  # [N, H, Dk, Dv] fp32 or None
    cu_seqlens: torch.Tensor | None = None  # int32 [N+1] on the same device, packed inputs


def _fill_block(g, nt, H, Dk, Dv, qkv_dtype, shift, alpha_one, device):
    q = torch.randn(nt, H, Dk, generator=g, device=device, dtype=torch.float64)
    k = torch.randn(nt, H, Dk, generator=g, device=device, dtype=torch.float64)
    v = torch.randn(nt, H, Dv, generator=g, device=device, dtype=torch.float64)
    z = torch.randn(nt, H, Dk, generator=g, device=device, dtype=torch.float64)
    zb = torch.randn(nt, H, generator=g, device=device, dtype=torch.float64)
    q = q / torch.linalg.vector_norm(q, dim=-1, keepdim=True)
    k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)
    if alpha_one:
        a = torch.ones_like(z)
    else:
        a = torch.exp(-_softplus64(z + shift))
    b = torch.sigmoid(zb)
    return (q.to(qkv_dtype), k.to(qkv_dtype), v.to(qkv_dtype), a.to(torch.float32),
            b.to(torch.float32))


def make_tokens(ntok: int, H: int, Dk: int, Dv: int, *, seed: int, qkv_dtype=torch.bfloat16,
                shift: float = 1.0, alpha_one: bool = False, device="cpu"):
    """Packed token tensors [ntok, H, .] drawn block by block."""
    q = torch.empty(ntok, H, Dk, dtype=qkv_dtype, device=device)
    k = torch.empty_like(q)
    v = torch.empty(ntok, H, Dv, dtype=qkv_dtype, device=device)
    a = torch.empty(ntok, H, Dk, dtype=torch.float32, device=device)
    b = torch.empty(ntok, H, dtype=torch.float32, device=device)
    for blk, t0 in enumerate(range(0, ntok, BLOCK)):
        nt = min(BLOCK, ntok - t0)
        g = _gen(device, seed * 1_000_003 + blk)
        q[t0:t0 + nt], k[t0:t0 + nt], v[t0:t0 + nt], a[t0:t0 + nt], b[t0:t0 + nt] = \
            _fill_block(g, nt, H, Dk, Dv, qkv_dtype, shift, alpha_one, device)
    return q, k, v, a, b


def make_state(n: int, H: int, Dk: int, Dv: int, *, seed: int, std: float = 0.02, device="cpu"):
    g = _gen(device, seed * 1_000_003 + 999_983)
    s = torch.randn(n, H, Dk, Dv, generator=g, device=device, dtype=torch.float64) * std
    return s.to(torch.float32)


def make_dense(B: int, T: int, H: int, Dk: int, Dv: int, *, seed: int, qkv_dtype=torch.bfloat16,
               shift: float = 1.0, alpha_one: bool = False, state_std: float | None = 0.02,
               device="cpu") -> KdaInputs:
    """Dense [B, T, H, .] inputs; batch b uses seed (seed, b)."""
    qs, ks, vs, as_, bs = [], [], [], [], []
    for bb in range(B):
        q, k, v, a, b = make_tokens(T, H, Dk, Dv, seed=seed * 7919 + bb, qkv_dtype=qkv_dtype,
                                    shift=shift, alpha_one=alpha_one, device=device)
        qs.append(q); ks.append(k); vs.append(v); as_.append(a); bs.append(b)
    st = None if state_std is None else make_state(B, H, Dk, Dv, seed=seed, std=state_std,
                                                     device=device)
    return KdaInputs(torch.stack(qs), torch.stack(ks), torch.stack(vs), torch.stack(as_),
                     torch.stack(bs), st)


def varlen_lengths(n: int, lo: int, hi: int, *, seed: int) -> list[int]:
    """n sequence lengths drawn uniformly from the integers lo..hi inclusive."""
    g = _gen("cpu", seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def make_varlen(lengths: list[int], H: int, Dk: int, Dv: int, *, seed: int,
                qkv_dtype=torch.bfloat16, shift: float = 1.0, state_std: float | None = 0.02,
                device="cpu") -> KdaInputs:
    """Packed [1, sum(lengths), H, .] inputs with int32 cu_seqlens; sequence i is
    drawn exactly as a dense B = 1 input of its own length with seed (seed, i), so
    a sequence's values do not depend on its neighbours in the batch."""
    qs, ks, vs, as_, bs = [], [], [], [], []
    for i, L in enumerate(lengths):
        q, k, v, a, b = make_tokens(L, H, Dk, Dv, seed=seed * 7919 + i, qkv_dtype=qkv_dtype,
                                    shift=shift, device=device)
        qs.append(q); ks.append(k); vs.append(v); as_.append(a); bs.append(b)
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    st = None if state_std is None else make_state(len(lengths), H, Dk, Dv, seed=seed,
                                                     std=state_std, device=device)
    return KdaInputs(torch.cat(qs)[None], torch.cat(ks)[None], torch.cat(vs)[None],
                     torch.cat(as_)[None], torch.cat(bs)[None], st,
                     torch.tensor(cu, dtype=torch.int32, device=device))


def make_gate(kind: str, lead: tuple, H: int, Dk: int, *, seed: int, shift: float = 1.0,
              device="cpu"):
    """Seeded decay tensor for a gate parametrization (see the module docstring):
    returns (gate, a_log) -- gate [*lead, H, Dk] fp32 ([*lead, H] for 'scalar',
    None for 'none'), a_log [H] fp32 for 'bounded', else None."""
    g = _gen(device, seed * 1_000_033 + 17)
    lead = tuple(lead)
    if kind == "none":
        return None, None
    if kind == "scalar":
        z = torch.randn(*lead, H, generator=g, device=device, dtype=torch.float64)
        return torch.exp(-_softplus64(z + shift)).to(torch.float32), None
    z = torch.randn(*lead, H, Dk, generator=g, device=device, dtype=torch.float64)
    if kind == "alpha":
        return torch.exp(-_softplus64(z + shift)).to(torch.float32), None
    if kind == "log":
        return (-_softplus64(z + shift)).to(torch.float32), None
    if kind == "bounded":
        a_log = torch.rand(H, generator=g, device=device, dtype=torch.float64) * 2.0 - 1.0
        return z.to(torch.float32), a_log.to(torch.float32)
    raise ValueError(f"unknown gate kind {kind!r}")


@dataclass
class LayerInputs:
    xq: torch.Tensor          # [B, T, H, Dk]
    xk: torch.Tensor          # [B, T, H, Dk]
    xv: torch.Tensor          # [B, T, H, Dv]
    g: torch.Tensor           # [B, T, H, Dv] output-gate logits
    wq: torch.Tensor          # [H, Dk, 4]
    wk: torch.Tensor          # [H, Dk, 4]
    wv: torch.Tensor          # [H, Dv, 4]
    conv_state: torch.Tensor  # [N, 3, H, 2 Dk + Dv]
    norm_w: torch.Tensor      # [Dv]


def make_layer(B: int, T: int, H: int, Dk: int, Dv: int, *, seed: int, n_state: int | None = None,
               dtype=torch.bfloat16, device="cpu") -> LayerInputs:
    """Seeded inputs of the layer's prologue and epilogue (see the module docstring)."""
    g = _gen(device, seed * 1_000_037 + 29)
    rn = lambda *sh: torch.randn(*sh, generator=g, device=device, dtype=torch.float64)  # noqa: E731
    N = B if n_state is None else n_state
    return LayerInputs(
        rn(B, T, H, Dk).to(dtype), rn(B, T, H, Dk).to(dtype), rn(B, T, H, Dv).to(dtype),
        rn(B, T, H, Dv).to(dtype),
        (0.5 * rn(H, Dk, 4)).float(), (0.5 * rn(H, Dk, 4)).float(), (0.5 * rn(H, Dv, 4)).float(),
        rn(N, 3, H, 2 * Dk + Dv).float(),
        (torch.rand(Dv, generator=g, device=device, dtype=torch.float64) + 0.5).float())


# The workloads, named by what they are.
WORKLOADS = {
    "tiny_fp32": dict(B=1, T=256, H=2, D=64, qkv_dtype=torch.float32, shift=0.0,
                      state_std=None, seed=1001),
    "k3_prefill_8k": dict(B=1, T=8192, H=96, D=128, qkv_dtype=torch.bfloat16, shift=1.0,
                          state_std=0.02, seed=1002),
    "decode_b64": dict(B=64, T=1, H=96, D=128, qkv_dtype=torch.bfloat16, shift=1.0,
                       state_std=0.02, seed=1003),
    "varlen_16": dict(N=16, lo=1024, hi=16384, H=96, D=128, qkv_dtype=torch.bfloat16,
                      shift=1.0, state_std=0.02, seed=1004),
    "long_1m": dict(B=1, T=1_048_576, H=96, D=128, qkv_dtype=torch.bfloat16, shift=1.0,
                    state_std=0.02, seed=1005),
    # one device's share of the 8K layer when its 96 heads are split over 8
    # devices (heads are independent, so each holds 12 whole heads)
    "k3_prefill_8k_h12": dict(B=1, T=8192, H=12, D=128, qkv_dtype=torch.bfloat16, shift=1.0,
                              state_std=0.02, seed=1008),
}
