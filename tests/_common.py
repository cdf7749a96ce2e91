"""Shared helpers for the GPU parity tests (inputs come from the seeded generators;
expected values from the fp64 oracle only).

Every comparison is made twice: as one relative L2 error over the whole tensor,
and as the largest relative L2 error over its (sequence, head) buckets, so that
a short sequence or a single head cannot hide inside the norm of the rest
("Kimi Delta Attention 完全拆解", section "数值路径必须以 recurrent 版本为基准校验":
errors are to be read per bucket, not as one global figure).  Both must lie
within the workload's tolerance."""
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


def rounded(x, dtype):
    """The values x (fp64) takes when stored in the token dtype (one rounding to
    nearest even), back in fp64: the layer's prologue hands q, k and v to the
    recurrence in the token dtype, and the oracle's chain takes the same step."""
    return torch.as_tensor(np.asarray(x)).to(dtype).double().numpy()


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


# Bucket layouts: which axes name a bucket, and which are summed inside it.
#   "tokens"  [B, T, H, D]: one bucket per (b, h); with cu_seqlens (B = 1,
#             packed) one per (sequence, h), empty sequences skipped
#   "state"   [N, H, Dk, Dv]: one bucket per (n, h)
#   "step"    [B, H, D]: one per (b, h) (decode outputs)
#   "steps"   [B, N, H, D]: one per (b, h) over the N tokens (verify outputs)
def bucket_errors(x, ref, layout, cu=None):
    """Relative L2 error of each (sequence, head) bucket, as a flat array (a
    bucket whose reference is all zero contributes its absolute error)."""
    x, ref = _np(x), _np(ref)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    d2 = (x - ref) ** 2
    r2 = ref ** 2
    if layout == "tokens":
        if cu is not None:
            cu = [int(c) for c in (cu.cpu().tolist() if hasattr(cu, "cpu") else list(cu))]
            num = np.stack([d2[0, cu[i]:cu[i + 1]].sum(axis=(0, 2))
                            for i in range(len(cu) - 1) if cu[i + 1] > cu[i]])
            den = np.stack([r2[0, cu[i]:cu[i + 1]].sum(axis=(0, 2))
                            for i in range(len(cu) - 1) if cu[i + 1] > cu[i]])
        else:
            num, den = d2.sum(axis=(1, 3)), r2.sum(axis=(1, 3))
    elif layout == "state":
        num, den = d2.sum(axis=(2, 3)), r2.sum(axis=(2, 3))
    elif layout == "step":
        num, den = d2.sum(axis=2), r2.sum(axis=2)
    elif layout == "steps":
        num, den = d2.sum(axis=(1, 3)), r2.sum(axis=(1, 3))
    else:
        raise ValueError(f"unknown layout {layout!r}")
    num, den = np.sqrt(num.ravel()), np.sqrt(den.ravel())
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def close(x, ref, tol, layout, cu=None):
    """Asserts that the global relative L2 error and the largest per-bucket one
    are both within `tol`; returns (global, worst bucket)."""
    g = rel(x, ref)
    b = bucket_errors(x, ref, layout, cu)
    worst = float(b.max()) if b.size else 0.0
    assert g <= tol and worst <= tol, (f"rel-L2 {g:.3e}, worst (sequence, head) bucket "
                                       f"{worst:.3e} (bucket {int(b.argmax())}), tolerance {tol:.1e}")
    return g, worst
