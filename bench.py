"""KDA forward benchmark on one MI355X.

One step = one chunked prefill (every step of the chunk form) of a K3-shaped
layer: B=1, H=96, T=8192, d_k=d_v=128, bf16 q/k/v, fp32 alpha/beta/state,
fp32 output, inputs resident in HBM, in the schedule the library prefers for
the shape (two-pass: a first pass over all (chunk, head) items, then the
state pass; one kda_prefill_chunked call, two kernel launches, workspace
allocated once outside the timed region).  The line also carries the fused
single-kernel schedule's time on the same step, the decode step's state
bandwidth (64 sessions x 96 heads x 128x128 fp32 state, updated in place), a
speculative-decoding round on the same sessions (verify 8 draft tokens, commit
them), the step's roofline position, and the fp64 CPU oracle timed on this host
on the same prefill workload.

Also timed: the packed workload (16 sequences of seeded lengths in [1024, 16384],
one kda_prefill_varlen call) and the 1,048,576-token prefill (one call, inputs
generated on the device), each with its roofline position.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-long]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def prefill_bytes(B, T, H, Dk, Dv):
    """Algorithmic HBM bytes of one prefill launch: bf16 q, k, v; fp32 alpha,
    beta and o, per token-head; fp32 initial and final state per sequence-head."""
    per_token_head = 2 * Dk + 2 * Dk + 2 * Dv + 4 * Dk + 4 + 4 * Dv
    return B * T * H * per_token_head + 2 * B * H * Dk * Dv * 4


def prefill_flops(B, T, H, d, C=64):
    """The chunk kernel's FLOP count per head, 6 T d^2 + 3 T C d + T C^2
    ("Kimi Delta Attention 完全拆解", section "Prefill 仍是线性复杂度")."""
    return B * H * (6 * T * d * d + 3 * T * C * d + T * C * C)


def decode_bytes(B, H, Dk, Dv):
    state = 2 * B * H * Dk * Dv * 4
    other = B * H * (2 * Dk + 2 * Dk + 2 * Dv + 4 * Dk + 4 + 4 * Dv)
    return state, other


def measured_traffic(summary: str, sources: list[str]):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if kv.get("source_sha256") != h.hexdigest():
        return None
    return float(kv["traffic_bytes_per_launch"].split()[0])


def measured_mfma(summary: str, sources: list[str]):
    """Matrix-core counters of a committed rocprofv3 summary: busy fraction per
    kernel and hardware FLOPs per call, or None when the sources changed."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    kv, busy = {}, {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
            if key.strip().endswith("] busy_frac"):
                busy[key.strip()[1:key.index("]")]] = float(val.split()[0])
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if kv.get("source_sha256") != h.hexdigest():
        return None
    return {"busy_frac": busy, "hw_flops_per_call": float(kv["hw_flops_per_call"].split()[0])}


PREFILL_SOURCES = ["kimi_delta_attention_amd/csrc/kda_prefill.hip",
                   "kimi_delta_attention_amd/csrc/kda_prefill_prep.hip",
                   "kimi_delta_attention_amd/csrc/kda_prefill_state.hip",
                   "kimi_delta_attention_amd/csrc/kda_frag.h",
                   "kimi_delta_attention_amd/csrc/kda_common.h"]
DECODE_SOURCES = ["kimi_delta_attention_amd/csrc/kda_decode.hip",
                  "kimi_delta_attention_amd/csrc/kda_common.h",
                  "kimi_delta_attention_amd/csrc/kda_frag.h",
                  "kimi_delta_attention_amd/csrc/kda_layer.h"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 1,048,576-token prefill leg (its inputs take ~180 GB)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); "
              "the operator is not sharded across GPUs", file=sys.stderr)
        sys.exit(2)

    import torch

    import kimi_delta_attention_amd as kda
    from kimi_delta_attention_amd import synth

    d = torch.device("cuda:0")
    w = synth.WORKLOADS["k3_prefill_8k"]
    B, T, H, D = w["B"], w["T"], w["H"], w["D"]
    print(f"bench: generating k3_prefill_8k inputs B={B} T={T} H={H} d={D}", file=sys.stderr,
          flush=True)
    inp = synth.make_dense(B, T, H, D, D, seed=w["seed"], state_std=w["state_std"], device=d)
    o = torch.empty(B, T, H, D, dtype=torch.float32, device=d)
    fs = torch.empty(B, H, D, D, dtype=torch.float32, device=d)
    lib = kda.load()
    two_pass = bool(lib.kda_prefill_two_pass_preferred(1, B, B * T, H, D, D))
    schedule = "two_pass" if two_pass else "fused"
    ws = (torch.empty(kda.workspace_size(B, T, H, D, D), dtype=torch.uint8, device=d)
          if two_pass else None)

    def step(sched=schedule):
        kda.prefill_chunked(inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                            initial_state=inp.state, final_state=fs, o=o, schedule=sched,
                            workspace=ws if sched == "two_pass" else None)

    # plain device copy of known size: calibrates HBM byte counters under rocprofv3
    calib = torch.empty(64 << 20, dtype=torch.float32, device=d)  # 256 MiB
    calib2 = torch.empty_like(calib)
    calib2.copy_(calib)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(d)  # the library launches on this stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]  # ms per launch
    total_ms = ev[0].elapsed_time(ev[-1])
    ms_step = total_ms / args.steps
    avg_launch_ms = sum(per) / len(per)
    tokens_s = B * T * args.steps / (total_ms / 1e3)
    nbytes = prefill_bytes(B, T, H, D, D)
    gbs = nbytes / (avg_launch_ms / 1e3) / 1e9
    tflops = prefill_flops(B, T, H, D) / (avg_launch_ms / 1e3) / 1e12
    print(f"bench: prefill ({schedule}) {ms_step:.3f} ms/step, {gbs:.0f} GB/s algorithmic, "
          f"{tflops:.1f} TFLOP/s (pages' count), wall {wall:.2f}s", file=sys.stderr, flush=True)

    # the other schedule on the same step, for context (not the headline value)
    other = "fused" if two_pass else None
    other_ms = None
    if other:
        for _ in range(2):
            step(other)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step(other)
        e1.record(stream)
        torch.cuda.synchronize()
        other_ms = e0.elapsed_time(e1) / args.steps
        print(f"bench: prefill ({other}) {other_ms:.3f} ms/step", file=sys.stderr, flush=True)

    # decode step (state read + write once per step)
    wd = synth.WORKLOADS["decode_b64"]
    dec = synth.make_dense(wd["B"], 1, wd["H"], wd["D"], wd["D"], seed=wd["seed"],
                           state_std=wd["state_std"], device=d)
    dq, dk, dv, da, db = (x[:, 0].contiguous() for x in (dec.q, dec.k, dec.v, dec.alpha, dec.beta))
    st = dec.state
    od = torch.empty(wd["B"], wd["H"], wd["D"], dtype=torch.float32, device=d)
    for _ in range(5):
        kda.decode_step(dq, dk, dv, da, db, st, o=od)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.decode_steps):
        kda.decode_step(dq, dk, dv, da, db, st, o=od)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / args.decode_steps
    sbytes, obytes = decode_bytes(wd["B"], wd["H"], wd["D"], wd["D"])
    dec_state_gbs = sbytes / (dec_ms / 1e3) / 1e9
    dec_total_gbs = (sbytes + obytes) / (dec_ms / 1e3) / 1e9
    print(f"bench: decode {dec_ms * 1e3:.1f} us/step, state {dec_state_gbs:.0f} GB/s",
          file=sys.stderr, flush=True)

    # speculative round on the decode workload: verify NS draft tokens per session
    # (state read only), then commit all of them (state read and written once)
    NS = 8
    sp = synth.make_dense(wd["B"], NS, wd["H"], wd["D"], wd["D"], seed=wd["seed"] + 100,
                          state_std=wd["state_std"], device=d)
    osp = torch.empty(wd["B"], NS, wd["H"], wd["D"], dtype=torch.float32, device=d)
    nacc = torch.full((wd["B"],), NS, dtype=torch.int32, device=d)

    def verify():
        kda.decode_verify(sp.q, sp.k, sp.v, sp.alpha, sp.beta, sp.state, o=osp)

    def commit():
        kda.decode_commit(sp.k, sp.v, sp.alpha, sp.beta, nacc, sp.state)

    def timed(f, reps, warm=3):
        for _ in range(warm):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ver_ms = timed(verify, args.decode_steps)
    com_ms = timed(commit, args.decode_steps)
    rnd_ms = timed(lambda: (verify(), commit()), args.decode_steps)
    tok_in = NS * wd["B"] * wd["H"]  # token-heads per round
    dd = wd["D"]
    spec_bytes = (3 * sbytes // 2                               # state: read, read, write
                  + tok_in * (2 * dd * 3 + 4 * dd + 4 + 4 * dd)  # verify: q k v, alpha, beta, o
                  + tok_in * (2 * dd * 2 + 4 * dd + 4))          # commit: k v, alpha, beta
    print(f"bench: spec round N={NS}: verify {ver_ms * 1e3:.1f} us + commit {com_ms * 1e3:.1f} us"
          f" = {rnd_ms * 1e3:.1f} us ({NS * dec_ms / rnd_ms:.2f}x {NS} decode steps)",
          file=sys.stderr, flush=True)

    # the layer around the recurrence: the fused layer decode step (prologue +
    # step + epilogue in one kernel) against the three calls, and the standalone
    # prologue / epilogue over the prefill layer
    lay = synth.make_layer(wd["B"], 1, wd["H"], wd["D"], wd["D"], seed=wd["seed"] + 200,
                           device=d)
    lst, lcs = dec.state.clone(), lay.conv_state.clone()
    ly = torch.empty(wd["B"], 1, wd["H"], wd["D"], dtype=torch.bfloat16, device=d)
    layer_ms = timed(lambda: kda.decode_layer("step", lay.xq, lay.xk, lay.xv, lay.wq, lay.wk,
                                              lay.wv, lcs, dec.alpha, dec.beta, lst, lay.g,
                                              lay.norm_w, y=ly), args.decode_steps)
    lcs2 = torch.empty_like(lcs)
    g1 = lay.g[:, 0].contiguous()
    ly1 = torch.empty(wd["B"], wd["H"], wd["D"], dtype=torch.bfloat16, device=d)

    def composed():
        q1, k1, v1, _ = kda.prologue(lay.xq, lay.xk, lay.xv, lay.wq, lay.wk, lay.wv,
                                     conv_state=lcs, conv_state_out=lcs2)
        o1 = kda.decode_step(q1[:, 0], k1[:, 0], v1[:, 0], da, db, lst, o=od)
        kda.epilogue(o1, g1, lay.norm_w, y=ly1)

    comp_ms = timed(composed, args.decode_steps)
    pl = synth.make_layer(B, T, H, D, D, seed=w["seed"] + 300, device=d)
    pro_ms = timed(lambda: kda.prologue(pl.xq, pl.xk, pl.xv, pl.wq, pl.wk, pl.wv,
                                        conv_state=pl.conv_state), 10)
    py = torch.empty(B, T, H, D, dtype=torch.bfloat16, device=d)
    epi_ms = timed(lambda: kda.epilogue(o, pl.g, pl.norm_w, y=py), 10)
    # the whole layer over the prefill in one call (prologue inside the first
    # pass), against the standalone prologue, recurrence and epilogue composed
    pcs = torch.empty_like(pl.conv_state)
    lo_ = torch.empty(B, T, H, D, dtype=torch.float32, device=d)
    lay_ms = timed(lambda: kda.prefill_layer(pl.xq, pl.xk, pl.xv, pl.wq, pl.wk, pl.wv, inp.alpha,
                                             inp.beta, pl.g, pl.norm_w, conv_state=pl.conv_state,
                                             initial_state=inp.state, final_state=fs,
                                             conv_state_out=pcs, o=lo_, y=py, workspace=ws),
                   10)

    def layer_composed():
        q3, k3, v3, _ = kda.prologue(pl.xq, pl.xk, pl.xv, pl.wq, pl.wk, pl.wv,
                                     conv_state=pl.conv_state, conv_state_out=pcs)
        kda.prefill_chunked(q3, k3, v3, inp.alpha, inp.beta, initial_state=inp.state,
                            final_state=fs, o=lo_, schedule=schedule, workspace=ws)
        kda.epilogue(lo_, pl.g, pl.norm_w, y=py)

    lay_comp_ms = timed(layer_composed, 10)
    print(f"bench: layer decode step {layer_ms * 1e3:.1f} us fused vs {comp_ms * 1e3:.1f} us "
          f"composed; prefill prologue {pro_ms * 1e3:.1f} us, epilogue {epi_ms * 1e3:.1f} us; "
          f"layer prefill {lay_ms:.3f} ms in one call vs {lay_comp_ms:.3f} ms composed",
          file=sys.stderr, flush=True)

    # one device's share of the layer under an 8-way head split (12 heads): the
    # segmented two-pass schedule against the unsegmented one and the fused kernel
    wh = synth.WORKLOADS["k3_prefill_8k_h12"]
    hin = synth.make_dense(wh["B"], wh["T"], wh["H"], wh["D"], wh["D"], seed=wh["seed"],
                           state_std=wh["state_std"], device=d)
    hB, hT, hH, hD = wh["B"], wh["T"], wh["H"], wh["D"]
    nseg = kda.segments_preferred(torch.bfloat16, hB, hB * hT, hH, hD, hD)
    hws = torch.empty(kda.segmented_workspace_size(hB, hH, hD, hD, nseg), dtype=torch.uint8,
                      device=d)
    ho = torch.empty(hB, hT, hH, hD, dtype=torch.float32, device=d)
    hfs = torch.empty(hB, hH, hD, hD, dtype=torch.float32, device=d)
    hg = (hin.q, hin.k, hin.v, hin.alpha, hin.beta)
    seg_ms = timed(lambda: kda.prefill_segmented(*hg, initial_state=hin.state, n_segments=nseg,
                                                 final_state=hfs, o=ho, workspace=hws),
                   args.steps)
    h2p_ms = timed(lambda: kda.prefill_chunked(*hg, initial_state=hin.state, final_state=hfs,
                                               o=ho, schedule="two_pass", workspace=hws),
                   args.steps)
    hfu_ms = timed(lambda: kda.prefill_chunked(*hg, initial_state=hin.state, final_state=hfs,
                                               o=ho, schedule="fused"), args.steps)
    hbytes = prefill_bytes(hB, hT, hH, hD, hD)
    print(f"bench: 12-head share: segmented ({nseg}) {seg_ms:.3f} ms, two-pass {h2p_ms:.3f} ms, "
          f"fused {hfu_ms:.3f} ms", file=sys.stderr, flush=True)

    # the packed workload: 16 sequences of seeded lengths in [1024, 16384], one
    # kda_prefill_varlen call (two-pass, workspace allocated once)
    wv = synth.WORKLOADS["varlen_16"]
    vlen = synth.varlen_lengths(wv["N"], wv["lo"], wv["hi"], seed=wv["seed"])
    vin = synth.make_varlen(vlen, wv["H"], wv["D"], wv["D"], seed=wv["seed"], device=d)
    vtok, vH, vD, vN = sum(vlen), wv["H"], wv["D"], wv["N"]
    vo = torch.empty(1, vtok, vH, vD, dtype=torch.float32, device=d)
    vfs = torch.empty(vN, vH, vD, vD, dtype=torch.float32, device=d)
    vws = torch.empty(kda._lib.varlen_workspace_size(vN, vtok, vH, vD, vD), dtype=torch.uint8,
                      device=d)
    var_ms = timed(lambda: kda.prefill_varlen(vin.q, vin.k, vin.v, vin.alpha, vin.beta,
                                              vin.cu_seqlens, initial_state=vin.state,
                                              final_state=vfs, o=vo, schedule="two_pass",
                                              workspace=vws), max(3, args.steps // 5), warm=2)
    # per token-head as prefill_bytes, plus an initial and a final state per sequence
    var_bytes = vtok * vH * (2 * vD * 3 + 4 * vD + 4 + 4 * vD) + 2 * vN * vH * vD * vD * 4
    print(f"bench: varlen_16 ({vtok} tokens) {var_ms:.3f} ms, "
          f"{var_bytes / (var_ms / 1e3) / 1e9:.0f} GB/s algorithmic", file=sys.stderr, flush=True)
    varlen = {"workload": f"varlen_16: {vN} packed sequences, lengths seeded in [1024, 16384] "
                          f"({vtok} tokens), H={vH}, d={vD}, one kda_prefill_varlen call",
              "tokens": vtok, "ms_per_call": var_ms, "tokens_per_s": vtok / (var_ms / 1e3),
              "roofline": {"bound": "hbm", "achieved": var_bytes / (var_ms / 1e3) / 1e9,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": var_bytes / (var_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                           "algorithmic_bytes_per_call": var_bytes,
                           "floor_ms": var_bytes / (HBM_PEAK_GBS * 1e9) * 1e3}}
    del vin, vo, vfs, vws

    cpu = None
    if not args.no_cpu:
        import oracle
        nth = oracle.default_threads()
        print(f"bench: cpu oracle on the full prefill workload, {nth} threads", file=sys.stderr,
              flush=True)
        # inputs upcast to fp64 before the clock starts: the timed region is the
        # oracle's token loop alone; best of three passes
        host = [x.cpu().double().numpy() for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                                                    inp.state)]
        runs = []
        for _ in range(3):
            tc = time.perf_counter()
            oracle.recurrent(*host[:5], initial_state=host[5], nthreads=nth)
            runs.append(time.perf_counter() - tc)
        ct = min(runs)
        cpu = {"value": B * T / ct, "unit": "tokens/s", "cores": nth, "kind": "oracle",
               "sample": f"the whole workload (B={B}, T={T}, H={H}, d={D}): fp64 token loop over "
                         f"inputs already in fp64, best of 3 passes, {ct:.2f} s"}
        del host

    # the long-context workload: 1,048,576 tokens x 96 heads in one call (inputs
    # generated on the device, about 176 GB; 128 windows of 8192 tokens)
    long1m = None
    if not args.no_long:
        del inp, o, fs, ws, calib, calib2, dec, st, od, sp, osp, lay, lst, lcs, ly, ly1, lcs2, pl, \
            py, lo_, pcs, hin, hws, ho, hfs
        torch.cuda.empty_cache()
        wl = synth.WORKLOADS["long_1m"]
        free, _ = torch.cuda.mem_get_info(d)
        if free > 200e9:
            tg = time.perf_counter()
            lin = synth.make_dense(wl["B"], wl["T"], wl["H"], wl["D"], wl["D"], seed=wl["seed"],
                                   state_std=wl["state_std"], device=d)
            torch.cuda.synchronize()
            print(f"bench: long_1m inputs generated in {time.perf_counter() - tg:.1f} s",
                  file=sys.stderr, flush=True)
            lT, lH, lD = wl["T"], wl["H"], wl["D"]
            lo = torch.empty(1, lT, lH, lD, dtype=torch.float32, device=d)
            lfs = torch.empty(1, lH, lD, lD, dtype=torch.float32, device=d)
            lws = torch.empty(kda.workspace_size(1, lT, lH, lD, lD), dtype=torch.uint8, device=d)
            long_ms = timed(lambda: kda.prefill_chunked(lin.q, lin.k, lin.v, lin.alpha, lin.beta,
                                                        initial_state=lin.state, final_state=lfs,
                                                        o=lo, schedule="two_pass", workspace=lws),
                            3, warm=1)
            lbytes = prefill_bytes(1, lT, lH, lD, lD)
            print(f"bench: long_1m {long_ms:.2f} ms, {lbytes / (long_ms / 1e3) / 1e9:.0f} GB/s "
                  "algorithmic", file=sys.stderr, flush=True)
            long1m = {"workload": "long_1m: B=1, T=1,048,576, H=96, d=128, one "
                                  "kda_prefill_chunked call (two-pass, 128 windows)",
                      "ms_per_call": long_ms, "tokens_per_s": lT / (long_ms / 1e3),
                      "roofline": {"bound": "hbm", "achieved": lbytes / (long_ms / 1e3) / 1e9,
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": lbytes / (long_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                                   "algorithmic_bytes_per_call": lbytes,
                                   "floor_ms": lbytes / (HBM_PEAK_GBS * 1e9) * 1e3}}
            del lin, lo, lfs, lws
            torch.cuda.empty_cache()
        else:
            long1m = {"skipped": f"needs ~200 GB of device memory, {free / 1e9:.0f} GB free"}

    traffic = measured_traffic(f"prefill_{schedule}__k3_prefill_8k__hbm_counters.txt", PREFILL_SOURCES)
    mf = measured_mfma(f"prefill_{schedule}__k3_prefill_8k__mfma_counters.txt", PREFILL_SOURCES)
    line = {
        "metric": "KDA prefill tokens/s (H=96,d=128) + decode-step state GB/s vs HBM peak",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "k3_prefill_8k", "B": B, "T": T, "H": H, "d_k": D, "d_v": D,
                   "chunk": 64, "qkv": "bf16", "alpha_beta_state": "fp32", "o": "fp32",
                   "schedule": schedule},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "traffic_unit": "HBM bytes per kda_prefill_chunked call (rocprofv3 "
                                     "FETCH_SIZE + WRITE_SIZE of its kernels, copy-calibrated)",
                     "kernel": ("kda_prefill_chunked, two-pass: prefill_prep_kernel<128, 128, alpha gate> "
                                "+ prefill_state_kernel<128, 128>" if two_pass else
                                "kda_prefill_chunked, fused: prefill_bf16_kernel<128, fp32 out, alpha gate>"),
                     "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_ms": avg_launch_ms,
                     "traffic_gbps": (traffic / (avg_launch_ms / 1e3) / 1e9) if traffic else None,
                     "mfma_frac_pages_flops": tflops / BF16_PEAK_TFLOPS,
                     "mfma_counters": ({"busy_frac": mf["busy_frac"],
                                        "hw_tflops": mf["hw_flops_per_call"] / (avg_launch_ms / 1e3) / 1e12,
                                        "hw_frac_bf16_peak": mf["hw_flops_per_call"] / (avg_launch_ms / 1e3)
                                                             / 1e12 / BF16_PEAK_TFLOPS}
                                       if mf else None)},
        "prefill_other_schedule": ({"schedule": other, "ms_per_step": other_ms,
                                    "tokens_per_s": B * T / (other_ms / 1e3)} if other else None),
        "decode": {"workload": "decode_b64", "B": wd["B"], "H": wd["H"], "d": wd["D"],
                   "us_per_step": dec_ms * 1e3, "state_gbs": dec_state_gbs,
                   "total_gbs": dec_total_gbs,
                   "roofline": {"bound": "hbm", "achieved": dec_total_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": dec_total_gbs / HBM_PEAK_GBS,
                                "traffic": measured_traffic(
                                    "decode_kernel_step__decode_b64__hbm_counters.txt",
                                    DECODE_SOURCES)}},
        "spec_decode": {"workload": f"decode_b64, {NS} draft tokens per session, all accepted",
                        "N": NS, "verify_us": ver_ms * 1e3, "commit_us": com_ms * 1e3,
                        "us_per_round": rnd_ms * 1e3,
                        "tokens_per_s": NS * wd["B"] / (rnd_ms / 1e3),
                        "vs_single_steps": NS * dec_ms / rnd_ms,
                        "algorithmic_bytes_per_round": spec_bytes,
                        "roofline": {"bound": "hbm", "achieved": spec_bytes / (rnd_ms / 1e3) / 1e9,
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": spec_bytes / (rnd_ms / 1e3) / 1e9 / HBM_PEAK_GBS}},
        "layer": {"decode_step_fused_us": layer_ms * 1e3, "decode_step_composed_us": comp_ms * 1e3,
                  "decode_workload": "decode_b64: prologue (ShortConv 4 + Swish + L2Norm, conv "
                                     "state), step, RMSNorm x sigmoid gate; bf16 y",
                  "prefill_prologue_us": pro_ms * 1e3, "prefill_epilogue_us": epi_ms * 1e3,
                  "prefill_layer_ms": lay_ms, "prefill_layer_composed_ms": lay_comp_ms,
                  "prefill_workload": "k3_prefill_8k, standalone kernels (bf16 x, q/k/v, y; "
                                      "fp32 o)"},
        "prefill_one_device_share": {
            "workload": "k3_prefill_8k_h12: the 8K layer's 12 heads per device under an 8-way "
                        "head split (B=1, T=8192, d=128)",
            "segments": nseg, "segmented_ms": seg_ms, "two_pass_ms": h2p_ms, "fused_ms": hfu_ms,
            "tokens_per_s": hB * hT / (seg_ms / 1e3),
            "algorithmic_gbs": hbytes / (seg_ms / 1e3) / 1e9},
        "prefill_varlen_16": varlen,
        "prefill_long_1m": long1m,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
