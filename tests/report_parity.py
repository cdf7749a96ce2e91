"""Parity report of the HIP path against the fp64 oracle, as markdown: per
workload the global relative L2 error and the worst (sequence, head) bucket, then
the buckets grouped by sequence length, by decay range and by the final state's
norm ("Kimi Delta Attention 完全拆解", section "数值路径必须以 recurrent 版本为基准校验":
errors by length, gate range and state norm, not one global figure), and the
layer around the recurrence.  Not a pytest module; run on a GPU with
`python tests/report_parity.py [--long] > report.md`."""
import os
import random
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import kimi_delta_attention_amd as kda  # noqa: E402
import oracle  # noqa: E402
from kimi_delta_attention_amd import synth  # noqa: E402
from tests._common import TOL_BF16, TOL_F32, bucket_errors, oracle_heads, rounded  # noqa: E402

D = torch.device("cuda:0")
ROWS, BY_LEN, BY_DECAY, BY_NORM = [], [], [], []


def errs(x, ref, layout, cu=None):
    """(global rel-L2, per-bucket rel-L2 array)"""
    return oracle.rel_l2(x.cpu() if hasattr(x, "cpu") else x, ref), bucket_errors(x, ref, layout, cu)


def row(name, tol, o, s, note):
    (go, bo), (gs, bs) = o, s
    wo, ws = float(bo.max()), float(bs.max())
    ok = "ok" if max(go, gs, wo, ws) <= tol else "FAIL"
    ROWS.append(f"| {name} | {tol:.0e} | {go:.2e} | {wo:.2e} | {gs:.2e} | {ws:.2e} | {ok} | {note} |")
    print(f"report: {name}: o {go:.2e}/{wo:.2e}, S {gs:.2e}/{ws:.2e} {ok}", file=sys.stderr, flush=True)


def decay_row(name, alpha, bo, bs):
    """per-token -log alpha over all tokens and channels, and the smallest
    16-token tile decay product of any channel"""
    a = np.asarray(alpha, dtype=np.float64)
    nl = -np.log(a)
    q1, q50, q99 = np.percentile(nl, [1, 50, 99])
    T = a.shape[1]
    nt = T // 16
    tile = nl[:, :nt * 16].reshape(a.shape[0], nt, 16, *a.shape[2:]).sum(axis=2)
    BY_DECAY.append(f"| {name} | {q50:.3g} ({q1:.3g} .. {q99:.3g}) | e^-{tile.max():.1f} | "
                    f"{float(bo.max()):.2e} | {float(bs.max()):.2e} |")


def norm_rows(name, s_ref, bo, bs):
    """(sequence, head) buckets in quartiles of the oracle's final state norm"""
    nrm = np.linalg.norm(np.asarray(s_ref, dtype=np.float64), axis=(2, 3)).ravel()
    if bo.size != nrm.size:  # empty sequences have a state bucket but no token bucket
        return
    edges = np.quantile(nrm, [0, 0.25, 0.5, 0.75, 1.0])
    for i in range(4):
        m = (nrm >= edges[i]) & ((nrm <= edges[i + 1]) if i == 3 else (nrm < edges[i + 1]))
        BY_NORM.append(f"| {name} | Q{i + 1}: {edges[i]:.3g} .. {edges[i + 1]:.3g} | {int(m.sum())} | "
                       f"{float(bo[m].max()):.2e} | {float(bs[m].max()):.2e} |")


def heads_in_groups(inp, H, cu=None, group=24):
    """the oracle over every head, a group of heads at a time"""
    os_, ss = [], []
    for h0 in range(0, H, group):
        ro, rs = oracle_heads(inp, list(range(h0, min(H, h0 + group))), cu=cu)
        os_.append(ro)
        ss.append(rs)
    return np.concatenate(os_, axis=2), np.concatenate(ss, axis=1)


def dense(B, T, H, Dd, seed, **kw):
    return synth.make_dense(B, T, H, Dd, Dd, seed=seed, device=D, **kw)


def run(inp, schedule="auto", **kw):
    o, s = kda.prefill_chunked(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state,
                               schedule=schedule, **kw)
    torch.cuda.synchronize()
    return o, s


def main():
    t_start = time.time()
    # ---- tiny fp32
    w = synth.WORKLOADS["tiny_fp32"]
    inp = synth.make_dense(w["B"], w["T"], w["H"], w["D"], w["D"], seed=w["seed"],
                           qkv_dtype=w["qkv_dtype"], shift=w["shift"], state_std=None)
    o, s = kda.prefill_chunked(*(x.to(D) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)))
    ro, rs = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta)
    row("tiny_fp32 (B1 H2 T256 d64)", TOL_F32, errs(o, ro, "tokens"), errs(s, rs, "state"),
        "oracle, all heads")

    # ---- the 8K layer, both schedules, every head
    w = synth.WORKLOADS["k3_prefill_8k"]
    inp = dense(w["B"], w["T"], w["H"], w["D"], w["seed"], state_std=w["state_std"])
    ro, rs = heads_in_groups(inp, w["H"])
    for sched in ("two_pass", "fused"):
        o, s = run(inp, sched)
        eo, es = errs(o, ro, "tokens"), errs(s, rs, "state")
        row(f"k3_prefill_8k (B1 H96 T8192 d128), {sched}", TOL_BF16, eo, es, "oracle, all 96 heads")
    decay_row("k3_prefill_8k: the workloads' synthetic alpha", inp.alpha.cpu(), eo[1], es[1])
    norm_rows("k3_prefill_8k", rs, eo[1], es[1])

    # ---- the 12-head share, segmented
    w = synth.WORKLOADS["k3_prefill_8k_h12"]
    inp = dense(w["B"], w["T"], w["H"], w["D"], w["seed"], state_std=w["state_std"])
    ns = kda.segments_preferred(torch.bfloat16, w["B"], w["B"] * w["T"], w["H"], w["D"], w["D"])
    o, s = kda.prefill_segmented(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state,
                                 n_segments=ns)
    torch.cuda.synchronize()
    ro, rs = oracle_heads(inp, list(range(12)))
    row(f"k3_prefill_8k_h12 segmented x{ns} (B1 H12 T8192 d128)", TOL_BF16, errs(o, ro, "tokens"),
        errs(s, rs, "state"), "oracle, all 12 heads")

    # ---- decode step
    w = synth.WORKLOADS["decode_b64"]
    inp = synth.make_dense(w["B"], 1, w["H"], w["D"], w["D"], seed=w["seed"], state_std=0.02)
    st = inp.state.to(D)
    od = kda.decode_step(*(x[:, 0].to(D) for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)), st)
    ro, rs = oracle.recurrent(inp.q, inp.k, inp.v, inp.alpha, inp.beta, initial_state=inp.state)
    row("decode_b64 (B64 H96 d128)", TOL_BF16, errs(od, ro[:, 0], "step"), errs(st, rs, "state"),
        "oracle, all sessions and heads")

    # ---- varlen_16, every head; per-sequence buckets
    w = synth.WORKLOADS["varlen_16"]
    lengths = synth.varlen_lengths(w["N"], w["lo"], w["hi"], seed=w["seed"])
    inp = synth.make_varlen(lengths, w["H"], w["D"], w["D"], seed=w["seed"], device=D)
    o, s = kda.prefill_varlen(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.cu_seqlens,
                              initial_state=inp.state)
    torch.cuda.synchronize()
    cu = inp.cu_seqlens.cpu().numpy()
    ro, rs = heads_in_groups(inp, w["H"], cu=cu)
    eo, es = errs(o, ro, "tokens", cu), errs(s, rs, "state")
    row(f"varlen_16 (N16, {sum(lengths)} tokens, H96 d128)", TOL_BF16, eo, es,
        "oracle, all 96 heads, all sequences")
    bo, bs = eo[1].reshape(len(lengths), w["H"]), es[1].reshape(len(lengths), w["H"])
    for i in np.argsort(lengths):
        BY_LEN.append(f"| varlen_16 | {lengths[i]} | {bo[i].max():.2e} | {bs[i].max():.2e} |")
    norm_rows("varlen_16", rs, eo[1], es[1])

    # ---- packed edges: empty, one-token, shorter than a tile, window-crossing
    lengths = [3000, 0, 2, 70, 8192 + 500, 1, 130, 17]
    inp = synth.make_varlen(lengths, 4, 128, 128, seed=1400, device=D)
    cu = inp.cu_seqlens.cpu().numpy()
    ro, rs = oracle_heads(inp, list(range(4)), cu=cu)
    for sched in ("two_pass", "fused"):
        o, s = kda.prefill_varlen(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.cu_seqlens,
                                  initial_state=inp.state, schedule=sched)
        torch.cuda.synchronize()
        eo, es = errs(o, ro, "tokens", cu), errs(s, rs, "state")
        row(f"packed edges {lengths} (H4 d128), {sched}", TOL_BF16, eo, es, "oracle, all heads")
    nz = [L for L in lengths if L > 0]
    bo = eo[1].reshape(len(nz), 4)
    bs = es[1].reshape(len(lengths), 4)
    j = 0
    for i, L in enumerate(lengths):
        if L == 0:
            BY_LEN.append(f"| packed edges | 0 | - | {bs[i].max():.2e} |")
            continue
        BY_LEN.append(f"| packed edges | {L} | {bo[j].max():.2e} | {bs[i].max():.2e} |")
        j += 1

    # ---- decay regimes and gate parametrizations
    regimes = []
    inp = dense(1, 4096, 8, 128, 77, shift=-4.0)
    regimes.append(("slow decay (shift -4)", inp, None, None))
    inp = dense(1, 4096, 8, 128, 77, alpha_one=True)
    regimes.append(("alpha = 1", inp, None, None))
    inp = dense(1, 4096, 8, 128, 80)
    g = torch.Generator().manual_seed(81)
    inp.alpha = torch.exp(-(6.0 + 0.5 * torch.randn(inp.alpha.shape, generator=g,
                                                     dtype=torch.float64))).float().to(D)
    regimes.append(("fast decay (-log alpha ~ N(6, 0.5^2))", inp, None, None))
    for kind in ("log", "bounded", "scalar", "none"):
        inp = dense(1, 4096, 8, 128, 78)
        gate, a_log = synth.make_gate(kind, (1, 4096), 8, 128, seed=79, device=D)
        regimes.append((f"gate '{kind}'", inp, gate, a_log))
    for name, inp, gate, a_log in regimes:
        kind = name.split("'")[1] if name.startswith("gate") else "alpha"
        gt = inp.alpha if kind == "alpha" else gate
        o, s = kda.prefill_chunked(inp.q, inp.k, inp.v, gt, inp.beta, initial_state=inp.state,
                                   gate=kind, a_log=a_log)
        torch.cuda.synchronize()
        alpha = (inp.alpha.cpu().numpy() if kind == "alpha" else
                 oracle.gate_alpha(kind, None if gate is None else gate.cpu().numpy(), inp.q.shape,
                                   a_log=None if a_log is None else a_log.cpu().numpy()))
        ro, rs = oracle.recurrent(inp.q.cpu(), inp.k.cpu(), inp.v.cpu(), alpha, inp.beta.cpu(),
                                  initial_state=inp.state.cpu())
        eo, es = errs(o, ro, "tokens"), errs(s, rs, "state")
        row(f"{name} (B1 H8 T4096 d128)", TOL_BF16, eo, es,
            "oracle, all heads" + ("" if kind == "alpha" else "; fed the oracle's alpha of the gate"))
        decay_row(name, alpha, eo[1], es[1])

    # ---- speculative round
    B, N, H, Dd = 64, 8, 96, 128
    inp = synth.make_dense(B, N, H, Dd, Dd, seed=1006, device=D)
    z, a_log = synth.make_gate("bounded", (B, N), H, Dd, seed=1007, device=D)
    st = inp.state.clone()
    o = kda.decode_verify(inp.q, inp.k, inp.v, z, inp.beta, st, gate="bounded", a_log=a_log)
    n_acc = torch.randint(0, N + 1, (B,), generator=torch.Generator().manual_seed(1008),
                          dtype=torch.int32)
    kda.decode_commit(inp.k, inp.v, z, inp.beta, n_acc.to(D), st, gate="bounded", a_log=a_log)
    torch.cuda.synchronize()
    alpha = oracle.gate_alpha("bounded", z.cpu().numpy(), inp.q.shape, a_log=a_log.cpu().numpy())
    hq, hk, hv, hb = (x.cpu() for x in (inp.q, inp.k, inp.v, inp.beta))
    ro, _ = oracle.recurrent(hq, hk, hv, alpha, hb, initial_state=inp.state.cpu())
    lens = [int(x) for x in n_acc]
    sel = lambda x: torch.cat([torch.as_tensor(x)[b, :lens[b]] for b in range(B)])[None]  # noqa: E731
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    _, rs = oracle.recurrent(sel(hq), sel(hk), sel(hv), sel(alpha), sel(hb), cu_seqlens=cu,
                             initial_state=inp.state.cpu())
    row("spec round (B64 H96 d128, 8 drafts, bounded gate)", TOL_BF16, errs(o, ro, "steps"),
        errs(st, rs, "state"), "oracle: verify outputs, committed states (seeded prefixes)")

    # ---- the layer: prologue, recurrence and epilogue against the oracle's chain
    f = lambda x: x.float().cpu()  # noqa: E731
    w = synth.WORKLOADS["k3_prefill_8k"]
    B, T, H, Dd = 1, 8192, 96, 128
    L = synth.make_layer(B, T, H, Dd, Dd, seed=1360, device=D)
    r = synth.make_dense(B, T, H, Dd, Dd, seed=1361, state_std=0.02, device=D)
    y, o, s, cs = kda.prefill_layer(L.xq, L.xk, L.xv, L.wq, L.wk, L.wv, r.alpha, r.beta, L.g,
                                    L.norm_w, conv_state=L.conv_state, initial_state=r.state)
    torch.cuda.synchronize()
    ys, oss, sss = [], [], []
    for h0 in range(0, H, 24):
        hs = list(range(h0, h0 + 24))
        sl = lambda x: f(x[:, :, hs])  # noqa: E731
        rq, rk, rv, _ = oracle.prologue(sl(L.xq), sl(L.xk), sl(L.xv), L.wq[hs].cpu(), L.wk[hs].cpu(),
                                        L.wv[hs].cpu(), state=L.conv_state[:, :, hs].cpu())
        rq, rk, rv = (rounded(x, torch.bfloat16) for x in (rq, rk, rv))
        ro, rs = oracle.recurrent(rq, rk, rv, r.alpha[:, :, hs].cpu().numpy(), r.beta[:, :, hs].cpu(),
                                  initial_state=r.state[:, hs].cpu())
        ys.append(oracle.rmsnorm_gate(ro, sl(L.g), L.norm_w.cpu()))
        oss.append(ro)
        sss.append(rs)
    ry, ro, rs = (np.concatenate(x, axis=a) for x, a in ((ys, 2), (oss, 2), (sss, 1)))
    row("layer prefill, one call (k3_prefill_8k): o", TOL_BF16, errs(o, ro, "tokens"),
        errs(s, rs, "state"), "oracle chain (prologue, q k v in bf16, recurrence), all 96 heads")
    row("layer prefill, one call (k3_prefill_8k): y", TOL_BF16, errs(y, ry, "tokens"),
        errs(s, rs, "state"), "oracle chain with the RMSNorm and gate, all 96 heads")

    if "--long" in sys.argv:
        w = synth.WORKLOADS["long_1m"]
        inp = dense(w["B"], w["T"], w["H"], w["D"], w["seed"], state_std=w["state_std"])
        o, s = run(inp)
        heads = sorted(random.Random(w["seed"]).sample(range(w["H"]), 4))
        t0 = time.time()
        ro, rs = oracle_heads(inp, heads)
        row("long_1m (B1 H96 T1048576 d128)", TOL_BF16, errs(o[:, :, heads], ro, "tokens"),
            errs(s[:, heads], rs, "state"), f"oracle, heads {heads} ({time.time() - t0:.0f}s)")

    print("# Parity against the fp64 oracle\n")
    print(f"Made by `python tests/report_parity.py{' --long' if '--long' in sys.argv else ''}` on one "
          f"MI355X ({time.time() - t_start:.0f} s).  Errors are relative L2: over the whole tensor "
          "(global) and over each (sequence, head) bucket (worst); a row passes when all four are "
          "within its tolerance.\n")
    print("| workload | tol | o global | o worst bucket | S global | S worst bucket | | compared against |")
    print("|---|---|---|---|---|---|---|---|")
    print("\n".join(ROWS))
    print("\n## By sequence length\n\nWorst (sequence, head) bucket of each sequence over its heads.\n")
    print("| workload | tokens | o worst head | S worst head |\n|---|---|---|---|")
    print("\n".join(BY_LEN))
    print("\n## By decay range\n\n-log alpha per token and channel: median (1st .. 99th percentile); "
          "the strongest decay of one channel over a 16-token tile; worst buckets.\n")
    print("| input | -log alpha | strongest tile decay | o worst bucket | S worst bucket |\n|---|---|---|---|---|")
    print("\n".join(BY_DECAY))
    print("\n## By state norm\n\nThe (sequence, head) buckets in quartiles of the oracle's final "
          "state norm ||S||_F; worst bucket in each.\n")
    print("| workload | ||S||_F range | buckets | o worst | S worst |\n|---|---|---|---|---|")
    print("\n".join(BY_NORM))


if __name__ == "__main__":
    main()
