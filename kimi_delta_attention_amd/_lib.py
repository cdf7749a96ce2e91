"""ctypes binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: tensors are passed as device pointers with their
sizes, on torch's current HIP stream; every step of the operator runs in the
library's HIP kernels.  There is no fallback: if the library is missing or
cannot be loaded, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_HIP"}

EXPORTED = ("kda_prefill_chunked", "kda_prefill_chunked_noalloc", "kda_prefill_varlen",
            "kda_decode_step",
            "kda_prefill_chunked_gated", "kda_prefill_varlen_gated", "kda_decode_step_gated",
            "kda_decode_verify", "kda_decode_commit", "kda_prologue", "kda_epilogue",
            "kda_decode_layer", "kda_prefill_layer", "kda_prefill_segmented",
            "kda_prefill_segmented_workspace_size", "kda_prefill_segments_preferred",
            "kda_prefill_workspace_size", "kda_prefill_varlen_workspace_size",
            "kda_prefill_two_pass_preferred", "kda_status_string", "kda_last_error_message")

SCHEDULES = ("auto", "fused", "two_pass")

# kda_gate_kind: how the decay tensor passed as `alpha` is read (include/kda.h)
GATES = {"alpha": 0, "log": 1, "bounded": 2, "scalar": 3, "none": 4}


class _Conv(ctypes.Structure):
    _fields_ = [("w_q", ctypes.c_void_p), ("w_k", ctypes.c_void_p), ("w_v", ctypes.c_void_p),
                ("eps", ctypes.c_float)]


class _OutGate(ctypes.Structure):
    _fields_ = [("g", ctypes.c_void_p), ("w", ctypes.c_void_p), ("eps", ctypes.c_float)]


DECODE_MODES = {"step": 0, "verify": 1, "commit": 2}


class _Gate(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("gate", ctypes.c_void_p),
                ("a_log", ctypes.c_void_p), ("g_min", ctypes.c_float)]


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Loads libkda.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python kimi_delta_attention_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_prefill_chunked.argtypes = [P, P, P, I, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.kda_prefill_chunked.restype = I
    lib.kda_prefill_chunked_noalloc.argtypes = [P, P, P, I, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.kda_prefill_chunked_noalloc.restype = I
    lib.kda_prefill_varlen.argtypes = [P, P, P, I, P, P, P, I, I, P, P, P, I, I, I, I, I, P, Z, P]
    lib.kda_prefill_varlen.restype = I
    lib.kda_decode_step.argtypes = [P, P, P, I, P, P, P, P, I, I, I, I, I, P]
    lib.kda_decode_step.restype = I
    G = ctypes.POINTER(_Gate)
    lib.kda_prefill_chunked_gated.argtypes = [P, P, P, I, G, P, P, P, P, I, I, I, I, I, I, I, P,
                                              Z, P]
    lib.kda_prefill_chunked_gated.restype = I
    lib.kda_prefill_varlen_gated.argtypes = [P, P, P, I, G, P, P, I, I, P, P, P, I, I, I, I, I,
                                             P, Z, P]
    lib.kda_prefill_varlen_gated.restype = I
    lib.kda_decode_step_gated.argtypes = [P, P, P, I, G, P, P, P, I, I, I, I, I, P]
    lib.kda_decode_step_gated.restype = I
    lib.kda_decode_verify.argtypes = [P, P, P, I, G, P, P, P, I, I, I, I, I, I, P]
    lib.kda_decode_verify.restype = I
    lib.kda_decode_commit.argtypes = [P, P, I, G, P, P, P, I, I, I, I, I, P]
    lib.kda_decode_commit.restype = I
    C = ctypes.POINTER(_Conv)
    lib.kda_prologue.argtypes = [P, P, P, I, C, P, P, P, I, I, I, I, I, P, P, P, P]
    lib.kda_prologue.restype = I
    lib.kda_epilogue.argtypes = [P, I, P, I, P, ctypes.c_float, P, I, ctypes.c_longlong, I, I, P]
    lib.kda_epilogue.restype = I
    lib.kda_decode_layer.argtypes = [I, P, P, P, I, C, P, G, P, P, ctypes.POINTER(_OutGate), P, I,
                                     P, I, I, I, I, I, P]
    lib.kda_decode_layer.restype = I
    lib.kda_prefill_segmented.argtypes = [P, P, P, I, G, P, P, I, I, P, P, P, I, I, I, I, I, I,
                                          P, Z, P]
    lib.kda_prefill_layer.argtypes = [P, P, P, I, C, P, P, G, P, P, I, I, P, P, P,
                                      ctypes.POINTER(_OutGate), P, I, I, I, I, I, I, P, Z, P]
    lib.kda_prefill_layer.restype = I
    lib.kda_prefill_segmented.restype = I
    lib.kda_prefill_segmented_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.kda_prefill_segmented_workspace_size.restype = Z
    lib.kda_prefill_segments_preferred.argtypes = [I, I, I, I, I, I]
    lib.kda_prefill_segments_preferred.restype = I
    lib.kda_prefill_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.kda_prefill_workspace_size.restype = Z
    lib.kda_prefill_varlen_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.kda_prefill_varlen_workspace_size.restype = Z
    lib.kda_prefill_two_pass_preferred.argtypes = [I, I, I, I, I, I]
    lib.kda_prefill_two_pass_preferred.restype = I
    lib.kda_status_string.argtypes = [I]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error_message.argtypes = []
    lib.kda_last_error_message.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load().kda_last_error_message().decode()
        raise KdaError(status, msg)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _out(t: torch.Tensor, name: str, shape: tuple, dtypes: tuple, device):
    """A caller-supplied output: a contiguous device tensor on `device` of exactly
    `shape` and one of `dtypes` (the kernels write it through a raw pointer)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    _need(t, name, None, device)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    return t


_FLOAT_OUT = (torch.float32, torch.bfloat16)
_F32 = (torch.float32,)


def _final_state(final_state, shape, dev):
    if isinstance(final_state, torch.Tensor):
        return _out(final_state, "final_state", shape, _F32, dev)
    if final_state:
        return torch.empty(shape, dtype=torch.float32, device=dev)
    return None


def _gate(kind: str, alpha, a_log, g_min: float, lead: tuple, H: int, Dk: int, dev):
    """Checks the decay tensor against its gate kind and returns the kda_gate
    descriptor.  Per-channel kinds take [*lead, H, Dk], 'scalar' [*lead, H],
    'none' no tensor; 'bounded' also takes a_log [H]."""
    if kind not in GATES:
        raise ValueError(f"gate must be one of {tuple(GATES)}")
    if kind == "none":
        if alpha is not None:
            raise ValueError("gate 'none' takes no decay tensor (pass alpha=None)")
        return _Gate(GATES[kind], None, None, 0.0)
    _need(alpha, "alpha", torch.float32, dev)
    want = (*lead, H) if kind == "scalar" else (*lead, H, Dk)
    if tuple(alpha.shape) != want:
        raise ValueError(f"gate '{kind}' expects a decay tensor of shape {want}, "
                         f"got {tuple(alpha.shape)}")
    al = None
    if kind == "bounded":
        if a_log is None:
            raise ValueError("gate 'bounded' needs a_log [H]")
        _need(a_log, "a_log", torch.float32, dev)
        if tuple(a_log.shape) != (H,):
            raise ValueError("a_log must be [H]")
        al = a_log.data_ptr()
    return _Gate(GATES[kind], alpha.data_ptr(), al, float(g_min))


def workspace_size(B: int, T: int, H: int, Dk: int, Dv: int, chunk: int = 64) -> int:
    return int(load().kda_prefill_workspace_size(B, T, H, Dk, Dv, chunk))


def varlen_workspace_size(N: int, total_tokens: int, H: int, Dk: int, Dv: int,
                          chunk: int = 64) -> int:
    return int(load().kda_prefill_varlen_workspace_size(N, total_tokens, H, Dk, Dv, chunk))


def _workspace(schedule, workspace, dtype, n_seq, tokens, size, dev):
    """The workspace argument for the requested schedule: None (fused) or a
    uint8 device tensor of at least `size` bytes (two-pass).  'auto' asks the
    library which schedule it expects to be faster."""
    if schedule not in SCHEDULES:
        raise ValueError(f"schedule must be one of {SCHEDULES}")
    if schedule == "fused":
        return None
    H, Dk, Dv = size[2], size[3], size[4]
    if schedule == "auto" and not load().kda_prefill_two_pass_preferred(
            _DT[dtype], n_seq, tokens, H, Dk, Dv):
        return None
    need = size[0]
    if need == 0:  # nothing to split (no tokens) or no two-pass kernel for the shape
        return None
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
        return workspace
    return torch.empty(need, dtype=torch.uint8, device=dev)


_DT = {torch.bfloat16: KDA_BF16, torch.float32: KDA_F32}


def prefill_chunked(q, k, v, alpha, beta, initial_state=None, out_dtype=torch.float32,
                    final_state: bool | torch.Tensor = True, o: torch.Tensor | None = None,
                    schedule: str = "auto", workspace: torch.Tensor | None = None,
                    gate: str = "alpha", a_log: torch.Tensor | None = None,
                    g_min: float = -5.0):
    """Dense chunked prefill.  q, k, alpha [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H];
    initial_state [B,H,Dk,Dv] fp32 or None.  schedule: 'auto', 'fused' or
    'two_pass' (the latter with `workspace`, a uint8 device buffer, or one
    allocated here).  gate: how `alpha` is read -- 'alpha' (the decay itself),
    'log' (log alpha), 'bounded' (logits z with a_log [H] and g_min), 'scalar'
    (one alpha per token and head, [B,T,H]) or 'none' (alpha = 1, pass None).
    Returns (o, final_state)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    g = _gate(gate, alpha, a_log, g_min, (B, T), H, Dk, dev)
    _need(beta, "beta", torch.float32, dev)
    if k.shape != q.shape or v.shape != (B, T, H, Dv) or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if initial_state.shape != (B, H, Dk, Dv):
            raise ValueError("initial_state must be [B, H, Dk, Dv]")
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=out_dtype, device=dev)
    else:
        _out(o, "o", (B, T, H, Dv), _FLOAT_OUT, dev)
    fs = _final_state(final_state, (B, H, Dk, Dv), dev)
    ws = _workspace(schedule, workspace, q.dtype, B, B * T,
                    (workspace_size(B, T, H, Dk, Dv), B, H, Dk, Dv), dev)
    _check(load().kda_prefill_chunked_gated(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), ctypes.byref(g), _ptr(beta), _ptr(initial_state),
        _ptr(fs), _ptr(o), _dt(o), B, T, H, Dk, Dv, 64, _ptr(ws),
        0 if ws is None else ws.numel(), _stream(dev)))
    return o, fs


def prefill_chunked_noalloc(q, k, v, alpha, beta, initial_state=None,
                            final_state: bool | torch.Tensor = True,
                            o: torch.Tensor | None = None, out_dtype=torch.float32):
    """kda_prefill_chunked_noalloc: the dense prefill with its workspace in the
    library's device array (nothing allocated by the library; with `o` and a
    `final_state` tensor given, nothing allocated here either).  Tensors as for
    prefill_chunked.  Returns (o, final_state)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(alpha, "alpha", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, T, H, Dv) \
            or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if initial_state.shape != (B, H, Dk, Dv):
            raise ValueError("initial_state must be [B, H, Dk, Dv]")
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=out_dtype, device=dev)
    else:
        _out(o, "o", (B, T, H, Dv), _FLOAT_OUT, dev)
    fs = _final_state(final_state, (B, H, Dk, Dv), dev)
    _check(load().kda_prefill_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(alpha), _ptr(beta), _ptr(initial_state),
        _ptr(fs), _ptr(o), _dt(o), B, T, H, Dk, Dv, 64, _stream(dev)))
    return o, fs


def prefill_varlen(q, k, v, alpha, beta, cu_seqlens, initial_state=None,
                   out_dtype=torch.float32, final_state: bool | torch.Tensor = True,
                   o: torch.Tensor | None = None, schedule: str = "auto",
                   workspace: torch.Tensor | None = None, gate: str = "alpha",
                   a_log: torch.Tensor | None = None, g_min: float = -5.0):
    """Packed prefill.  q, k, alpha [1,NTOK,H,Dk]; v [1,NTOK,H,Dv]; beta [1,NTOK,H];
    cu_seqlens int32 [N+1] on the device; states [N,H,Dk,Dv].  schedule,
    workspace and the gate arguments as for prefill_chunked.  Returns
    (o, final_state)."""
    _, NT, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    if q.shape[0] != 1:
        raise ValueError("packed inputs have B == 1")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    if k.shape != q.shape or v.shape != (1, NT, H, Dv) or beta.shape != (1, NT, H):
        raise ValueError("inconsistent shapes")
    g = _gate(gate, alpha, a_log, g_min, (1, NT), H, Dk, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be [N + 1]")
    N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if initial_state.shape != (N, H, Dk, Dv):
            raise ValueError("initial_state must be [N, H, Dk, Dv]")
    if o is None:
        o = torch.empty(1, NT, H, Dv, dtype=out_dtype, device=dev)
    else:
        _out(o, "o", (1, NT, H, Dv), _FLOAT_OUT, dev)
    fs = _final_state(final_state, (N, H, Dk, Dv), dev)
    ws = _workspace(schedule, workspace, q.dtype, N, NT,
                    (varlen_workspace_size(N, NT, H, Dk, Dv), N, H, Dk, Dv), dev)
    _check(load().kda_prefill_varlen_gated(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), ctypes.byref(g), _ptr(beta), _ptr(cu_seqlens), N, NT,
        _ptr(initial_state), _ptr(fs), _ptr(o), _dt(o), H, Dk, Dv, 64, _ptr(ws),
        0 if ws is None else ws.numel(), _stream(dev)))
    return o, fs


MAX_SEGMENTS = 16


def segmented_workspace_size(n_seq: int, H: int, Dk: int, Dv: int, n_segments: int) -> int:
    return int(load().kda_prefill_segmented_workspace_size(n_seq, H, Dk, Dv, 64, n_segments))


def segments_preferred(dtype, n_seq: int, tokens: int, H: int, Dk: int, Dv: int) -> int:
    return int(load().kda_prefill_segments_preferred(_DT[dtype], n_seq, tokens, H, Dk, Dv))


def prefill_segmented(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None,
                      n_segments: int | None = None, out_dtype=torch.float32,
                      final_state: bool | torch.Tensor = True, o: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, gate: str = "alpha",
                      a_log: torch.Tensor | None = None, g_min: float = -5.0):
    """Two-pass prefill with each window's chunks of a sequence split into up to
    n_segments segments that run side by side (None: the library's choice).
    Dense (cu_seqlens None): tensors as for prefill_chunked; packed: as for
    prefill_varlen.  bf16 q, k, v.  Returns (o, final_state)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    _need(beta, "beta", torch.float32, dev)
    if k.shape != q.shape or v.shape != (B, T, H, Dv) or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed inputs have B == 1")
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        n_seq, tokens = cu_seqlens.numel() - 1, T
    else:
        n_seq, tokens = B, B * T
    g = _gate(gate, alpha, a_log, g_min, (B, T), H, Dk, dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if initial_state.shape != (n_seq, H, Dk, Dv):
            raise ValueError("initial_state must be [n_seq, H, Dk, Dv]")
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=out_dtype, device=dev)
    else:
        _out(o, "o", (B, T, H, Dv), _FLOAT_OUT, dev)
    fs = _final_state(final_state, (n_seq, H, Dk, Dv), dev)
    if n_segments is None:
        n_segments = segments_preferred(q.dtype, n_seq, tokens, H, Dk, Dv)
    need = segmented_workspace_size(n_seq, H, Dk, Dv, n_segments)
    if need == (1 << 64) - 1:
        raise ValueError(f"n_segments must lie in [1, {MAX_SEGMENTS}]")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    _check(load().kda_prefill_segmented(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), ctypes.byref(g), _ptr(beta), _ptr(cu_seqlens), n_seq,
        T if cu_seqlens is None else tokens, _ptr(initial_state), _ptr(fs), _ptr(o), _dt(o), H, Dk,
        Dv, 64, n_segments, _ptr(workspace), workspace.numel(), _stream(dev)))
    return o, fs


def decode_step(q, k, v, alpha, beta, state, out_dtype=torch.float32,
                o: torch.Tensor | None = None, gate: str = "alpha",
                a_log: torch.Tensor | None = None, g_min: float = -5.0):
    """One token per session.  q, k, alpha [B,H,Dk]; v [B,H,Dv]; beta [B,H];
    state [B,H,Dk,Dv] fp32 updated in place; the gate arguments as for
    prefill_chunked ('scalar' takes alpha [B,H]).  Returns o [B,H,Dv]."""
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    g = _gate(gate, alpha, a_log, g_min, (B,), H, Dk, dev)
    _need(beta, "beta", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    if state.shape != (B, H, Dk, Dv) or beta.shape != (B, H):
        raise ValueError("inconsistent shapes")
    if o is None:
        o = torch.empty(B, H, Dv, dtype=out_dtype, device=dev)
    else:
        _out(o, "o", (B, H, Dv), _FLOAT_OUT, dev)
    _check(load().kda_decode_step_gated(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), ctypes.byref(g), _ptr(beta), _ptr(state), _ptr(o),
        _dt(o), B, H, Dk, Dv, _stream(dev)))
    return o


MAX_DRAFT = 16  # tokens per session of one verify / commit call


def _multi_inputs(k, v, alpha, beta, gate, a_log, g_min, q=None):
    B, N, H, Dk = k.shape
    Dv = v.shape[-1]
    dev = k.device
    for t, n in ((k, "k"), (v, "v")) + (((q, "q"),) if q is not None else ()):
        _need(t, n, k.dtype, dev)
    if (q is not None and q.shape != k.shape) or v.shape != (B, N, H, Dv):
        raise ValueError("inconsistent shapes")
    g = _gate(gate, alpha, a_log, g_min, (B, N), H, Dk, dev)
    _need(beta, "beta", torch.float32, dev)
    if beta.shape != (B, N, H):
        raise ValueError("beta must be [B, N, H]")
    return B, N, H, Dk, Dv, dev, g


def decode_verify(q, k, v, alpha, beta, state, out_dtype=torch.float32,
                  o: torch.Tensor | None = None, gate: str = "alpha",
                  a_log: torch.Tensor | None = None, g_min: float = -5.0):
    """Speculative-decoding verify: N draft tokens per session stepped from
    `state` (read only).  q, k, alpha [B,N,H,Dk]; v [B,N,H,Dv]; beta [B,N,H];
    state [B,H,Dk,Dv] fp32; gate arguments as for prefill_chunked.  Returns
    o [B,N,H,Dv], token t's output after tokens 0..t (bitwise the steps' below 6
    drafts; from 6 on the chunk form, equal up to fp32 rounding)."""
    B, N, H, Dk, Dv, dev, g = _multi_inputs(k, v, alpha, beta, gate, a_log, g_min, q=q)
    _need(state, "state", torch.float32, dev)
    if state.shape != (B, H, Dk, Dv):
        raise ValueError("state must be [B, H, Dk, Dv]")
    if o is None:
        o = torch.empty(B, N, H, Dv, dtype=out_dtype, device=dev)
    else:
        _out(o, "o", (B, N, H, Dv), _FLOAT_OUT, dev)
    _check(load().kda_decode_verify(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), ctypes.byref(g), _ptr(beta), _ptr(state), _ptr(o),
        _dt(o), B, N, H, Dk, Dv, _stream(dev)))
    return o


def decode_commit(k, v, alpha, beta, n_accept, state, gate: str = "alpha",
                  a_log: torch.Tensor | None = None, g_min: float = -5.0):
    """Speculative-decoding commit: replays tokens 0..n_accept[b]-1 of the same
    draft inputs into `state` in place (bitwise what that many decode_step calls
    leave below 12 drafts; from 12 drafts on the library takes the chunk form,
    equal up to fp32 rounding).  n_accept: int32 [B] device tensor, clamped to
    [0, N] on the device."""
    B, N, H, Dk, Dv, dev, g = _multi_inputs(k, v, alpha, beta, gate, a_log, g_min)
    _need(state, "state", torch.float32, dev)
    _need(n_accept, "n_accept", torch.int32, dev)
    if state.shape != (B, H, Dk, Dv) or n_accept.shape != (B,):
        raise ValueError("state must be [B, H, Dk, Dv] and n_accept [B]")
    _check(load().kda_decode_commit(
        _ptr(k), _ptr(v), _dt(k), ctypes.byref(g), _ptr(beta), _ptr(n_accept), _ptr(state),
        B, N, H, Dk, Dv, _stream(dev)))
    return state


def _conv(wq, wk, wv, eps, H, Dk, Dv, dev):
    for t, n, D in ((wq, "w_q", Dk), (wk, "w_k", Dk), (wv, "w_v", Dv)):
        _need(t, n, torch.float32, dev)
        if tuple(t.shape) != (H, D, 4):
            raise ValueError(f"{n} must be [H, {D}, 4]")
    return _Conv(wq.data_ptr(), wk.data_ptr(), wv.data_ptr(), float(eps))


def prologue(xq, xk, xv, wq, wk, wv, conv_state=None, cu_seqlens=None, eps: float = 1e-6,
             conv_state_out: bool | torch.Tensor = True):
    """The layer's prologue over a prefill: q, k = L2Norm(Swish(ShortConv(x))),
    v = Swish(ShortConv(x_v)).  xq, xk [B,T,H,Dk], xv [B,T,H,Dv] (packed: B = 1
    with cu_seqlens int32 [N+1]); taps wq, wk [H,Dk,4], wv [H,Dv,4] fp32;
    conv_state [N,3,H,2Dk+Dv] fp32 or None (zeros).  Returns (q, k, v,
    conv_state_out or None)."""
    B, T, H, Dk = xq.shape
    Dv = xv.shape[-1]
    dev = xq.device
    for t, n in ((xq, "x_q"), (xk, "x_k"), (xv, "x_v")):
        _need(t, n, xq.dtype, dev)
    if xk.shape != xq.shape or xv.shape != (B, T, H, Dv):
        raise ValueError("inconsistent shapes")
    c = _conv(wq, wk, wv, eps, H, Dk, Dv, dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed inputs have B == 1")
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    sw = (N, 3, H, 2 * Dk + Dv)
    if conv_state is not None:
        _need(conv_state, "conv_state", torch.float32, dev)
        if tuple(conv_state.shape) != sw:
            raise ValueError(f"conv_state must be {sw}")
    if isinstance(conv_state_out, torch.Tensor):
        so = _out(conv_state_out, "conv_state_out", sw, _F32, dev)
    elif conv_state_out:
        so = torch.empty(sw, dtype=torch.float32, device=dev)
    else:
        so = None
    q, k, v = torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv)
    _check(load().kda_prologue(
        _ptr(xq), _ptr(xk), _ptr(xv), _dt(xq), ctypes.byref(c), _ptr(conv_state), _ptr(so),
        _ptr(cu_seqlens), N, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _stream(dev)))
    return q, k, v, so


def epilogue(o, g, w, eps: float = 1e-5, out_dtype=None, y: torch.Tensor | None = None):
    """y = RMSNorm(o) * w * Sigmoid(g) per head: o, g [..., H, Dv]; w [Dv] fp32."""
    dev = o.device
    _need(o, "o", None, dev)
    _need(g, "g", None, dev)
    _need(w, "w", torch.float32, dev)
    if g.shape != o.shape or o.dim() < 2 or tuple(w.shape) != (o.shape[-1],):
        raise ValueError("o and g must match, w must be [Dv]")
    H, Dv = o.shape[-2], o.shape[-1]
    tokens = o.numel() // (H * Dv)
    if y is None:
        y = torch.empty(o.shape, dtype=out_dtype or o.dtype, device=dev)
    else:
        _out(y, "y", tuple(o.shape), _FLOAT_OUT, dev)
    _check(load().kda_epilogue(_ptr(o), _dt(o), _ptr(g), _dt(g), _ptr(w), float(eps), _ptr(y),
                               _dt(y), tokens, H, Dv, _stream(dev)))
    return y



def decode_layer(mode: str, xq, xk, xv, wq, wk, wv, conv_state, alpha, beta, state, g=None,
                 norm_w=None, n_accept=None, gate: str = "alpha",
                 a_log: torch.Tensor | None = None, g_min: float = -5.0, conv_eps: float = 1e-6,
                 norm_eps: float = 1e-5, out_dtype=torch.float32, y: torch.Tensor | None = None):
    """The fused recurrent layer step: prologue (conv taps wq, wk [H,Dk,4], wv
    [H,Dv,4], conv_state [B,3,H,2Dk+Dv]), the decode call of `mode` ('step' with
    N = 1, 'verify', 'commit' with n_accept), epilogue (g [B,N,H,Dv], norm_w
    [Dv]).  xq, xk [B,N,H,Dk], xv [B,N,H,Dv] are the projections' outputs.
    Returns y [B,N,H,Dv] (None for commit); state and conv_state are updated in
    place by step and commit.  Bitwise prologue + the plain call (fp32 o) +
    epilogue: the fused verify and commit take the plain calls' forms."""
    if mode not in DECODE_MODES:
        raise ValueError(f"mode must be one of {tuple(DECODE_MODES)}")
    B, N, H, Dk, Dv, dev, gd = _multi_inputs(xk, xv, alpha, beta, gate, a_log, g_min, q=xq)
    c = _conv(wq, wk, wv, conv_eps, H, Dk, Dv, dev)
    _need(conv_state, "conv_state", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    if tuple(conv_state.shape) != (B, 3, H, 2 * Dk + Dv) or state.shape != (B, H, Dk, Dv):
        raise ValueError("conv_state must be [B, 3, H, 2Dk+Dv] and state [B, H, Dk, Dv]")
    og = _OutGate(None, None, float(norm_eps))
    if mode == "commit":
        _need(n_accept, "n_accept", torch.int32, dev)
        if n_accept.shape != (B,):
            raise ValueError("n_accept must be [B]")
        y = None
    else:
        _need(g, "g", xq.dtype, dev)
        _need(norm_w, "norm_w", torch.float32, dev)
        if g.shape != (B, N, H, Dv) or tuple(norm_w.shape) != (Dv,):
            raise ValueError("g must be [B, N, H, Dv] and norm_w [Dv]")
        og = _OutGate(g.data_ptr(), norm_w.data_ptr(), float(norm_eps))
        if y is None:
            y = torch.empty(B, N, H, Dv, dtype=out_dtype, device=dev)
        else:
            _out(y, "y", (B, N, H, Dv), _FLOAT_OUT, dev)
    _check(load().kda_decode_layer(
        DECODE_MODES[mode], _ptr(xq), _ptr(xk), _ptr(xv), _dt(xq), ctypes.byref(c),
        _ptr(conv_state), ctypes.byref(gd), _ptr(beta), _ptr(state), ctypes.byref(og), _ptr(y),
        _dt(y) if y is not None else KDA_F32, _ptr(n_accept), B, N, H, Dk, Dv, _stream(dev)))
    return y


def prefill_layer(xq, xk, xv, wq, wk, wv, alpha, beta, g, norm_w, conv_state=None,
                  initial_state=None, cu_seqlens=None, n_segments: int = 1,
                  conv_eps: float = 1e-6, norm_eps: float = 1e-5, out_dtype=torch.float32,
                  final_state: bool | torch.Tensor = True,
                  conv_state_out: bool | torch.Tensor = True, o: torch.Tensor | None = None,
                  y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  gate: str = "alpha", a_log: torch.Tensor | None = None, g_min: float = -5.0):
    """The recurrent layer over a prefill: prologue (taps wq, wk [H,Dk,4], wv
    [H,Dv,4]; conv_state [N,3,H,2Dk+Dv] or None) fused into the two-pass first
    pass, the recurrence (n_segments as for prefill_segmented), the epilogue (g
    [..,H,Dv] bf16, norm_w [Dv]).  xq, xk [B,T,H,Dk], xv [B,T,H,Dv] bf16 (packed:
    B = 1 with cu_seqlens).  Returns (y, o, final_state, conv_state_out)."""
    B, T, H, Dk = xq.shape
    Dv = xv.shape[-1]
    dev = xq.device
    for t, n in ((xq, "x_q"), (xk, "x_k"), (xv, "x_v")):
        _need(t, n, xq.dtype, dev)
    if xk.shape != xq.shape or xv.shape != (B, T, H, Dv) or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    _need(beta, "beta", torch.float32, dev)
    c = _conv(wq, wk, wv, conv_eps, H, Dk, Dv, dev)
    gd = _gate(gate, alpha, a_log, g_min, (B, T), H, Dk, dev)
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed inputs have B == 1")
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        n_seq = cu_seqlens.numel() - 1
    else:
        n_seq = B
    sw = (n_seq, 3, H, 2 * Dk + Dv)
    if conv_state is not None:
        _need(conv_state, "conv_state", torch.float32, dev)
        if tuple(conv_state.shape) != sw:
            raise ValueError(f"conv_state must be {sw}")
    if isinstance(conv_state_out, torch.Tensor):
        so = _out(conv_state_out, "conv_state_out", sw, _F32, dev)
    elif conv_state_out:
        so = torch.empty(sw, dtype=torch.float32, device=dev)
    else:
        so = None
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if initial_state.shape != (n_seq, H, Dk, Dv):
            raise ValueError("initial_state must be [n_seq, H, Dk, Dv]")
    fs = _final_state(final_state, (n_seq, H, Dk, Dv), dev)
    _need(g, "g", xq.dtype, dev)
    _need(norm_w, "norm_w", torch.float32, dev)
    if g.shape != (B, T, H, Dv) or tuple(norm_w.shape) != (Dv,):
        raise ValueError("g must be [B, T, H, Dv] and norm_w [Dv]")
    og = _OutGate(g.data_ptr(), norm_w.data_ptr(), float(norm_eps))
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=torch.float32, device=dev)
    else:
        _out(o, "o", (B, T, H, Dv), _F32, dev)
    if y is None:
        y = torch.empty(B, T, H, Dv, dtype=out_dtype, device=dev)
    else:
        _out(y, "y", (B, T, H, Dv), _FLOAT_OUT, dev)
    need = segmented_workspace_size(n_seq, H, Dk, Dv, n_segments)
    if need == (1 << 64) - 1:
        raise ValueError(f"n_segments must lie in [1, {MAX_SEGMENTS}]")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    _check(load().kda_prefill_layer(
        _ptr(xq), _ptr(xk), _ptr(xv), _dt(xq), ctypes.byref(c), _ptr(conv_state), _ptr(so),
        ctypes.byref(gd), _ptr(beta), _ptr(cu_seqlens), n_seq, T if cu_seqlens is None else T,
        _ptr(initial_state), _ptr(fs), _ptr(o), ctypes.byref(og), _ptr(y), _dt(y), H, Dk, Dv, 64,
        n_segments, _ptr(workspace), workspace.numel(), _stream(dev)))
    return y, o, fs, so
