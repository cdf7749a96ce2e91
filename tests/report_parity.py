"""Prints the relative L2 error of the HIP path against the fp64 oracle for each
workload (and against the GPU decode replay for the full-size ones).  Not a
pytest module; run on a GPU with `python tests/report_parity.py [--long]`."""
import os
import random
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import kimi_delta_attention_amd as kda  # noqa: E402
import oracle  # noqa: E402
from kimi_delta_attention_amd import synth  # noqa: E402
from tests._common import oracle_heads  # noqa: E402


def row(name, tol, eo, es, note=""):
    ok = "ok" if max(eo, es) <= tol else "FAIL"
    print(f"| {name} | {tol:.0e} | {eo:.2e} | {es:.2e} | {ok} | {note} |", flush=True)


def replay(inp, o, s):
    state = inp.state.clone()
    T = inp.q.shape[1]
    orep = torch.empty_like(o)
    for t in range(T):
        kda.decode_step(inp.q[:, t], inp.k[:, t], inp.v[:, t], inp.alpha[:, t], inp.beta[:, t],
                        state, o=orep[:, t])
    torch.cuda.synchronize()
    return oracle.rel_l2(orep.cpu(), o.cpu()), oracle.rel_l2(state.cpu(), s.cpu())


def main():
    d = torch.device("cuda:0")
    print("| workload | tol | rel-L2 o | rel-L2 S | | compared against |")
    print("|---|---|---|---|---|---|")
    w = synth.WORKLOADS["tiny_fp32"]
    inp = synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                           qkv_dtype=w["qkv_dtype"], shift=w["shift"], state_std=None)
    o, s = kda.prefill_chunked(*(x.to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)))
    ro, rs = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta)
    row("tiny_fp32 (B1 H2 T256 d64)", 1e-5, oracle.rel_l2(o.cpu(), ro), oracle.rel_l2(s.cpu(), rs),
        "oracle, all heads")

    w = synth.WORKLOADS["k3_prefill_8k"]
    inp = synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                           state_std=w["state_std"], device=d)
    o, s = kda.prefill_chunked(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state)
    torch.cuda.synchronize()
    heads = list(range(0, 96, 12))
    ro, rs = oracle_heads(inp, heads)
    row("k3_prefill_8k (B1 H96 T8192 d128)", 2e-3, oracle.rel_l2(o[:, :, heads].cpu(), ro),
        oracle.rel_l2(s[:, heads].cpu(), rs), f"oracle, heads {heads}")
    eo, es = replay(inp, o, s)
    row("k3_prefill_8k", 2e-3, eo, es, "GPU decode replay, all 96 heads")

    w = synth.WORKLOADS["k3_prefill_8k_h12"]
    inp = synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                           state_std=w["state_std"], device=d)
    ns = kda.segments_preferred(torch.bfloat16, w["B"], w["B"] * w["T"], w["H"], w["D"], w["D"])
    o, s = kda.prefill_segmented(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                 initial_state=inp.state, n_segments=ns)
    torch.cuda.synchronize()
    ro, rs = oracle_heads(inp, list(range(12)))
    row(f"k3_prefill_8k_h12 segmented x{ns} (B1 H12 T8192 d128)", 2e-3,
        oracle.rel_l2(o.cpu(), ro), oracle.rel_l2(s.cpu(), rs), "oracle, all 12 heads")

    w = synth.WORKLOADS["decode_b64"]
    inp = synth.make_dense(w["B"], 1, w["H"], w["D"], w["D"], seed=w["seed"], state_std=0.02)
    st = inp.state.to(d)
    od = kda.decode_step(*(x[:, 0].to(d) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)), st)
    ro, rs = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state)
    row("decode_b64 (B64 H96 d128)", 2e-3, oracle.rel_l2(od.cpu(), ro[:, 0]),
        oracle.rel_l2(st.cpu(), rs), "oracle, all sessions and heads")

    w = synth.WORKLOADS["varlen_16"]
    lengths = synth.varlen_lengths(w["N"], w["lo"], w["hi"], seed=w["seed"])
    inp = synth.make_varlen(lengths, w["H"], w["D"], w["D"], seed=w["seed"], device=d)
    o, s = kda.prefill_varlen(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.cu_seqlens,
                              initial_state=inp.state)
    torch.cuda.synchronize()
    heads = [7, 40, 88]
    ro, rs = oracle_heads(inp, heads, cu=inp.cu_seqlens.cpu().numpy())
    row(f"varlen_16 (N16, {sum(lengths)} tokens, H96 d128)", 2e-3,
        oracle.rel_l2(o[:, :, heads].cpu(), ro), oracle.rel_l2(s[:, heads].cpu(), rs),
        f"oracle, heads {heads}, all sequences")

    for kind, shift, a1 in (("slow decay", -4.0, False), ("alpha=1", 1.0, True)):
        inp = synth.make_dense(1, 4096, 8, 128, 128, seed=77, shift=shift, alpha_one=a1, device=d)
        o, s = kda.prefill_chunked(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                   initial_state=inp.state)
        torch.cuda.synchronize()
        ro, rs = oracle_heads(inp, list(range(8)))
        row(f"{kind} (B1 H8 T4096 d128)", 2e-3, oracle.rel_l2(o.cpu(), ro),
            oracle.rel_l2(s.cpu(), rs), "oracle, all heads (stress input)")

    for kind in ("log", "bounded", "scalar", "none"):
        inp = synth.make_dense(1, 4096, 8, 128, 128, seed=78, device=d)
        gate, a_log = synth.make_gate(kind, (1, 4096), 8, 128, seed=79, device=d)
        o, s = kda.prefill_chunked(inp.q, inp.k, inp.v, gate, inp.beta, initial_state=inp.state,
                                   gate=kind, a_log=a_log)
        torch.cuda.synchronize()
        alpha = oracle.gate_alpha(kind, None if gate is None else gate.cpu().numpy(), inp.q.shape,
                                  a_log=None if a_log is None else a_log.cpu().numpy())
        ro, rs = oracle.recurrent(inp.q.cpu(), inp.k.cpu(), inp.v.cpu(), alpha, inp.beta.cpu(),
                                  initial_state=inp.state.cpu())
        row(f"gate '{kind}' (B1 H8 T4096 d128)", 2e-3, oracle.rel_l2(o.cpu(), ro),
            oracle.rel_l2(s.cpu(), rs), "oracle fed the oracle's own alpha of the gate, all heads")

    # speculative round: verify 8 draft tokens per session, commit a seeded prefix
    B, N, H, D = 64, 8, 96, 128
    inp = synth.make_dense(B, N, H, D, D, seed=1006, device=d)
    z, a_log = synth.make_gate("bounded", (B, N), H, D, seed=1007, device=d)
    st = inp.state.clone()
    o = kda.decode_verify(inp.q, inp.k, inp.v, z, inp.beta, st, gate="bounded", a_log=a_log)
    n_acc = torch.randint(0, N + 1, (B,), generator=torch.Generator().manual_seed(1008),
                          dtype=torch.int32)
    kda.decode_commit(inp.k, inp.v, z, inp.beta, n_acc.to(d), st, gate="bounded", a_log=a_log)
    torch.cuda.synchronize()
    alpha = oracle.gate_alpha("bounded", z.cpu().numpy(), inp.q.shape, a_log=a_log.cpu().numpy())
    hq, hk, hv, hb = (x.cpu() for x in (inp.q, inp.k, inp.v, inp.beta))
    ro, _ = oracle.recurrent(hq, hk, hv, alpha, hb, initial_state=inp.state.cpu())
    lens = [int(x) for x in n_acc]
    sel = lambda x: torch.cat([torch.as_tensor(x)[b, :lens[b]] for b in range(B)])[None]  # noqa: E731
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    _, rs = oracle.recurrent(sel(hq), sel(hk), sel(hv), sel(alpha), sel(hb), cu_seqlens=cu,
                             initial_state=inp.state.cpu())
    row("spec round (B64 H96 d128, 8 drafts, bounded gate)", 2e-3, oracle.rel_l2(o.cpu(), ro),
        oracle.rel_l2(st.cpu(), rs), "oracle: verify outputs, committed states (seeded prefixes)")

    if "--long" in sys.argv:
        w = synth.WORKLOADS["long_1m"]
        inp = synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                               state_std=w["state_std"], device=d)
        o, s = kda.prefill_chunked(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                   initial_state=inp.state)
        torch.cuda.synchronize()
        heads = sorted(random.Random(w["seed"]).sample(range(w["H"]), 4))
        t0 = time.time()
        ro, rs = oracle_heads(inp, heads)
        row("long_1m (B1 H96 T1048576 d128)", 2e-3, oracle.rel_l2(o[:, :, heads].cpu(), ro),
            oracle.rel_l2(s[:, heads].cpu(), rs), f"oracle, heads {heads} ({time.time()-t0:.0f}s)")


if __name__ == "__main__":
    main()
