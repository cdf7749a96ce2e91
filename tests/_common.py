"""Shared helpers for the GPU parity tests (inputs come from the seeded generators;
expected values from the fp64 oracle only)."""
import numpy as np
import torch

import oracle

TOL_F32 = 1e-5    # fp32 inputs, fp32 output
TOL_BF16 = 2e-3   # bf16 q/k/v, fp32 alpha/beta/state/accumulation, fp32 output
# bf16 output: one extra RNE rounding of o.  bf16 keeps 8 significant bits, so
# a rounding to nearest is off by at most 2^-8 relative per element (and so in
# relative L2)
TOL_BF16_OUT = TOL_BF16 + 2.0 ** -8


def dev():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to(x, d):
    return None if x is None else x.to(d)


def oracle_heads(inp, heads, cu=None):
    """Runs the oracle on a subset of heads; returns (o [B,T,len(heads),Dv], S [N,len(heads),Dk,Dv])."""
    sel = lambda t: t[:, :, heads].cpu()  # noqa: E731
    st = None if inp.state is None else inp.state[:, heads].cpu()
    return oracle.recurrent(sel(inp.q), sel(inp.k), sel(inp.v), sel(inp.alpha),
                            inp.beta[:, :, heads].cpu(), cu_seqlens=cu, initial_state=st)


def rel(x, ref):
    return oracle.rel_l2(x, ref)
