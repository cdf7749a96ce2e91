"""kda_prefill_chunked_noalloc, the prefill entry point that allocates nothing
(its two-pass workspace is a device array of the library), called through the
C ABI and compared with kda_prefill_chunked given a caller's workspace: the
same kernels in the same schedule, so the results must be bitwise equal.  Two
calls in a row, the second smaller, so that the second runs over what the
first left in the shared array."""
import ctypes

import pytest
import torch

import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import _lib, synth
from tests._common import dev

pytestmark = pytest.mark.gpu

OK, INVALID = 0, 1


def _noalloc(inp, o, fs, dtype=_lib.KDA_BF16):
    B, T, H, Dk = inp.q.shape
    Dv = inp.v.shape[-1]
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(inp.q.device).cuda_stream)
    return kda.load().kda_prefill_chunked_noalloc(
        p(inp.q), p(inp.k), p(inp.v), dtype, p(inp.alpha), p(inp.beta), p(inp.state), p(fs),
        p(o), _lib.KDA_F32, B, T, H, Dk, Dv, 64, stream)


def _one(case, d):
    B, T, H, D, dt = case
    inp = synth.make_dense(B, T, H, D, D, seed=1500 + T, qkv_dtype=dt, state_std=0.02, device=d)
    o = torch.full((B, T, H, D), float("nan"), dtype=torch.float32, device=d)
    fs = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device=d)
    st = _noalloc(inp, o, fs, _lib.KDA_BF16 if dt == torch.bfloat16 else _lib.KDA_F32)
    assert st == OK, kda.load().kda_last_error_message()
    ref_o, ref_s = kda.prefill_chunked(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                       initial_state=inp.state,
                                       schedule="two_pass" if dt == torch.bfloat16 else "auto")
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(fs, ref_s), case


def test_noalloc_equals_the_workspace_entry_point_on_consecutive_calls():
    d = dev()
    for case in ((1, 3000, 4, 128, torch.bfloat16),   # 47 chunks, 4 heads
                 (1, 700, 2, 64, torch.bfloat16),     # smaller, over the first call's leftovers
                 (1, 150, 2, 64, torch.float32)):     # fp32 inputs: no workspace at all
        _one(case, d)
    # twice the same call: bitwise reproducible
    inp = synth.make_dense(1, 9000, 2, 128, 128, seed=1510, state_std=0.02, device=d)
    outs = []
    for _ in range(2):
        o = torch.empty(1, 9000, 2, 128, dtype=torch.float32, device=d)
        fs = torch.empty(1, 2, 128, 128, dtype=torch.float32, device=d)
        assert _noalloc(inp, o, fs) == OK
        outs.append((o, fs))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_noalloc_rejects_sizes_beyond_its_scratch():
    d = dev()
    inp = synth.make_dense(1, 64, 16, 128, 128, seed=1520, state_std=0.02, device=d)
    o = torch.empty(1, 64, 16, 128, dtype=torch.float32, device=d)
    fs = torch.empty(1, 16, 128, 128, dtype=torch.float32, device=d)
    assert kda.workspace_size(1, 64, 16, 128, 128) > (128 << 20)
    assert _noalloc(inp, o, fs) == INVALID
    assert b"device scratch" in kda.load().kda_last_error_message()
