#!/usr/bin/env python3
"""Benchmark of the chunked gated delta-rule backward on one MI355X.

One step = one whole backward (forward recompute + backward, all kernels, the
fused entry point gdr_fwd_bwd) over the headline workload: GDN scalar gate,
B=1, T=32768, H=16, Dk=Dv=128, bf16 inputs, h0/dht ~ N(0, 0.1), synthetic
seeded inputs already resident in HBM.  Prints one JSON line.

ms_per_step is the median of the per-step times (a HIP event recorded after
every step on the stream the library launches on).  Every kernel is then timed
alone the same way (median over --stage-iters launches).  The roofline record
is the dominant kernel's bf16 MFMA fraction (algorithmic FLOPs of the chunked
method over its event-timed duration, against the 2.5 PFLOP/s dense peak),
with its HBM fraction beside it and, where rocprofv3 counter runs on the same
kernel sources exist, the counter-measured MFMA FLOPs and HBM bytes (and every
kernel's counter-measured MFMA fraction, with the combined fraction of the
recursions and the gradient kernel), plus the recursions' grid against the CUs
(the share of the device the reverse role can use).  The path
record is the roofline fraction of the whole step: the larger of its MFMA and
HBM floors (476.5 kFLOP and 1,800 B per token-head) over the measured time.
The float64 CPU oracle is timed on a bounded sample of the same workload (the
first --cpu-tokens tokens, all heads).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time
from typing import Dict

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from chunked_gated_delta_bwd_amd import binding as B  # noqa: E402
from chunked_gated_delta_bwd_amd import synth  # noqa: E402

GATE_NAMES = {0: "scalar", 1: "channel", 2: "channel_sigmoid"}
METRIC = "gated-delta-rule bwd tokens/s + ms/bwd at T=32k,H=16,D=128 bf16; MFMA %"
CSRC = os.path.join(ROOT, "chunked_gated_delta_bwd_amd", "csrc")
# Per-launch rocprofv3 counter readings (the summaries under profiles/), valid
# only for the kernel sources they were taken on:
# (workload, stage, sha256 prefix of the kernel sources) -> readings.
#   traffic:   HBM bytes, FETCH_SIZE and WRITE_SIZE scaled by a 1 GiB device copy
#   mfma_flop: SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (bf16 MFMA FLOPs)
MEASURED = {
    ("gdn_bf16_t32768_h16_d128", "prep", "3d8743f98324"): {'traffic': 716000000, 'mfma_flop': 19330000000},
    ("gdn_bf16_t32768_h16_d128", "chain_both", "3d8743f98324"): {'traffic': 1690000000, 'mfma_flop': 180420000000},
    ("gdn_bf16_t32768_h16_d128", "grads", "3d8743f98324"): {'traffic': 2125000000, 'mfma_flop': 120260000000},
    ("kda_bf16_t32768_h16_d128", "prep", "3d8743f98324"): {'traffic': 1841000000, 'mfma_flop': 53690000000},
    ("kda_bf16_t32768_h16_d128", "chain_both", "3d8743f98324"): {'traffic': 2795000000, 'mfma_flop': 128850000000},
    ("kda_bf16_t32768_h16_d128", "grads", "3d8743f98324"): {'traffic': 3794000000, 'mfma_flop': 188980000000},
    ("kda_bf16_t32768_h16_d128", "finish", "3d8743f98324"): {'traffic': 4000000},
    ("gdn_bf16_t32768_h32_d128", "prep", "3d8743f98324"): {'traffic': 1447000000, 'mfma_flop': 38650000000},
    ("gdn_bf16_t32768_h32_d128", "chain_both", "3d8743f98324"): {'traffic': 3385000000, 'mfma_flop': 360840000000},
    ("gdn_bf16_t32768_h32_d128", "grads", "3d8743f98324"): {'traffic': 4548000000, 'mfma_flop': 240520000000},
    ("gdn_gqa4_bf16_t32768_h32_d128", "prep", "3d8743f98324"): {'traffic': 1003000000, 'mfma_flop': 38650000000},
    ("gdn_gqa4_bf16_t32768_h32_d128", "chain_both", "3d8743f98324"): {'traffic': 2783000000, 'mfma_flop': 360840000000},
    ("gdn_gqa4_bf16_t32768_h32_d128", "grads", "3d8743f98324"): {'traffic': 4025000000, 'mfma_flop': 240520000000},
    ("gdn_gqa4_bf16_t32768_h32_d128", "finish", "3d8743f98324"): {'traffic': 672000000},
    ("gdn_bf16_t32768_h2_d128", "prep", "3d8743f98324"): {'traffic': 86000000, 'mfma_flop': 2420000000},
    ("gdn_bf16_t32768_h2_d128", "chain_both", "3d8743f98324"): {'traffic': 317000000, 'mfma_flop': 56830000000},
    ("gdn_bf16_t32768_h2_d128", "grads", "3d8743f98324"): {'traffic': 246000000, 'mfma_flop': 15030000000},
}


def kernel_source_hash() -> str:
    """sha256 prefix over every kernel source (sorted by name)."""
    import hashlib

    hsh = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                hsh.update(name.encode() + b"\0" + f.read())
    return hsh.hexdigest()[:12]
C = 64
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def algorithmic_work(inp, stage: str):
    """(flops, bytes) one launch of `stage` must do on this problem.

    FLOPs are the chunked method's own contractions per (chunk, head), counting
    triangular products at half size; bytes are the HBM traffic the stage
    cannot avoid (inputs read, outputs written, its workspace in and out).
    With grouped heads q and k have Hk < H heads and are read once per key head
    (the value heads of a group share them through L2); dq and dk leave the
    gradient stages per value head and the group sums (in "finish") reduce them.
    """
    H, D = inp["H"], inp["K"]
    Hk = inp.get("Hk") or H
    NC = sum((L + C - 1) // C for L in inp["lengths"])
    tokens = inp["B"] * inp["T"]
    ch = NC * H
    gk = D if inp["gate"] != 0 else 1
    io = 2 if inp["dtype"] == "bf16" else 4
    f_prep = 4 * C * C * D + C ** 3 // 3
    f_fwd = 4 * C * D * D
    f_bwd = 6 * C * D * D + C * C * D
    f_grads = 6 * C * D * D + 9 * C * C * D
    # scalar gate with bf16 inputs: the recursions take the raw q, k rows and row
    # factors, and W = A Diag(fw) k is never formed (A, 64 x 64, replaces W, 64 x D)
    raw = inp["gate"] == 0 and inp["dtype"] == "bf16"
    wt = C * C * 2 if raw else C * D * 2
    if stage == "prep":
        # q, k, v, g, b in; Gamma, row scalars, A, P, U' (and W unless raw) out
        b = tokens * (2 * Hk * D * io + H * (D * io + (1 + gk) * io)) + ch * (C * gk * 4 + 2 * C * 4 + 2 * C * C * 2
                                                              + (1 if raw else 2) * C * D * 2)
        return ch * f_prep, b
    if stage == "chain_fwd":
        # W (or A), U', k in; S, U out
        return ch * f_fwd, ch * (wt + C * D * 2 + D * D * 2 + C * D * 2) + tokens * Hk * D * io
    if stage == "chain_bwd":
        # W (or A), P, q, k, dO in; dS, dU out
        return ch * f_bwd, ch * (wt + C * C * 2 + D * D * 2 + C * D * 2) + tokens * (2 * Hk + H) * D * io
    if stage == "chain_both":
        a, b = algorithmic_work(inp, "chain_fwd"), algorithmic_work(inp, "chain_bwd")
        return a[0] + b[0], a[1] + b[1]
    if stage == "output":
        # S_n, U, P and Qbar (or the raw q rows and row factors) in; o out
        b = ch * (D * D * 2 + C * D * 2 + C * C * 2 + (0 if raw else C * D * 2)) + tokens * (H + (Hk if raw else 0)) * D * io
        return ch * (2 * C * D * D + C * C * D), b
    if stage == "grads":
        # fused with the prepare-backward: S, dS, U, dU, A, Gamma, (1/|q|, 1/|k|, beta)
        # per chunk (and M, the parameter partial sums for the per-channel gate);
        # q, k, v, dO, the gate and the beta logit read, dq, dk, dv, dg, db written
        # per token
        b = (ch * (2 * D * D * 2 + 2 * C * D * 2 + C * C * 2 + C * gk * 4 + 3 * C * 4)
             + tokens * (2 * Hk * D * io + H * (5 * D * io + 2 * gk * io + 2 * io)))
        if inp["gate"] != 0:
            b += ch * (C * C * 2 + (1 + gk) * 4)
        return ch * f_grads, b
    if stage == "finish":
        b = 0
        if inp["gate"] != 0:
            # the per-head reduction of the dA_log, ddt_bias partial sums
            b = ch * (1 + gk) * 4 + H * (1 + gk) * 4
        if Hk < H:
            # group sums: dq, dk per value head in, per key head out
            b += tokens * 2 * (H + Hk) * D * io
        return 0, b
    raise KeyError(stage)


def time_calls(fn, iters: int):
    """Milliseconds of each of `iters` back-to-back calls: HIP events recorded
    between the calls on the current stream (the stream the library launches
    on), bracketed by device synchronisations."""
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(iters):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def host_cpu():
    """The host's logical CPU count, the CPUs this process may run on, and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return os.cpu_count() or 1, usable, model


def cpu_baseline(inp, tokens: int, backward: bool = True):
    """The float64 oracle on the first `tokens` tokens of the workload (all heads)."""
    import oracle  # test infrastructure: only this leg of the benchmark uses it

    sub = dict(inp)
    for key in ("q", "k", "v", "dO", "g", "b"):
        sub[key] = inp[key][:, :tokens].contiguous()
    sub["T"] = tokens
    if inp["N"] == inp["B"]:      # dense: the first tokens of every batch row
        sub["lengths"] = [tokens] * inp["B"]
        sub["cu_seqlens"] = torch.arange(inp["B"] + 1, dtype=torch.int64) * tokens
    else:                         # packed: cut the packed axis, sequences keep their own states
        cu = torch.clamp(inp["cu_seqlens"], max=tokens)
        sub["cu_seqlens"] = cu
        sub["lengths"] = [int(x) for x in (cu[1:] - cu[:-1])]
    threads = oracle.default_threads()
    oracle.run(sub, nthreads=threads, backward=backward)  # build/load outside the timed call
    t0 = time.perf_counter()
    oracle.run(sub, nthreads=threads, backward=backward)
    dt = time.perf_counter() - t0
    nproc, usable, model = host_cpu()
    # the oracle's threads take one (sequence, head) each: no more of them work than there are pairs
    used = min(threads, len(sub["lengths"]) * inp["H"])
    what = "token recurrence + adjoint" if backward else "token recurrence (forward only)"
    return {"value": tokens / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "seconds": round(dt, 3), "nproc": nproc, "cpus_usable": usable, "cpu_model": model,
            "sample": f"first {tokens} of {inp['T']} tokens, all {inp['H']} heads of the same workload; "
                      f"float64 {what}, {used} threads over (sequence, head)"}


def roofline(inp, workload: str, name: str, ms: float) -> Dict:
    """The roofline record of one kernel of the chunked method (prologue,
    recursions, gradients: dense 64 x 64 and 64 x D contractions, so the bound
    is the bf16 matrix cores): algorithmic FLOPs per launch over the measured
    duration against the dense bf16 peak.  The HBM fraction of its algorithmic
    bytes and, where a counter run on the same kernel sources exists, the
    counter-measured HBM bytes and MFMA FLOPs are reported beside it."""
    flops, nbytes = algorithmic_work(inp, name)
    secs = ms * 1e-3
    achieved = flops / secs / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    h = kernel_source_hash()
    m = MEASURED.get((workload, name, h), {})
    roof["traffic"] = m.get("traffic")
    roof["kernel"] = name
    roof["ms"] = round(ms, 4)
    roof["source_hash"] = h
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = nbytes
    roof["hbm_frac"] = round(nbytes / secs / 1e9 / PEAK_HBM_GBS, 4)
    if m.get("mfma_flop") is not None:
        roof["mfma_counter_flops"] = m["mfma_flop"]
        roof["mfma_counter_frac"] = round(m["mfma_flop"] / secs / 1e12 / PEAK_BF16_TFLOPS, 4)
    return roof


# The method's own work per token-head (chunk 64, K = V = 128): 476.5 kFLOP
# (forward recompute 6CK + 4KV + C^2/3, backward 18CK + 12KV + 4C^2 per token)
# and 1,800 B (q, k, v, dO, g, b read, dq, dk, dv, dg, db written, bf16).
def path_floors(inp):
    K, V = inp["K"], inp["V"]
    th = inp["B"] * inp["T"] * inp["H"]
    io = 2 if inp["dtype"] == "bf16" else 4
    flop = th * (6 * C * K + 4 * K * V + C * C / 3 + 18 * C * K + 12 * K * V + 4 * C * C)
    gk = K if inp["gate"] != 0 else 1
    Hk = inp.get("Hk") or inp["H"]
    tok = inp["B"] * inp["T"]
    # per key head: q, k read, dq, dk written (4 K); per value head: v, dO read and
    # dv written (3 V), the gate read and dg written (2 gk), the beta logit read and
    # db written (2)
    nbytes = tok * io * (2 * 2 * Hk * K + inp["H"] * (3 * V + 2 * gk + 2))
    return flop, nbytes


def path_record(inp, ms: float, kernels, workload: str) -> Dict:
    flop, nbytes = path_floors(inp)
    t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3
    rec = {"frac": round(max(t_mfma, t_hbm) / ms, 4), "mfma_floor_ms": round(t_mfma, 4),
           "hbm_floor_ms": round(t_hbm, 4), "algorithmic_flops": int(flop), "algorithmic_bytes": int(nbytes)}
    h = kernel_source_hash()
    traffic = [MEASURED.get((workload, n, h), {}).get("traffic") for n in kernels]
    if kernels and all(t is not None for t in traffic):
        rec["traffic"] = sum(traffic)
        rec["traffic_ratio"] = round(sum(traffic) / nbytes, 2)
    return rec


GPU_CUS = 256


def counters_per_kernel(workload: str, kernels: Dict, roof: Dict) -> None:
    """Where counter runs on these kernel sources exist: each kernel's counter-measured
    bf16 MFMA fraction (MFMA FLOPs issued per launch / its time / bf16 peak), and the
    combined fraction of the recursions and the gradient kernel."""
    h = kernel_source_hash()
    for name, rec in kernels.items():
        m = MEASURED.get((workload, name, h), {})
        if m.get("mfma_flop") is not None:
            rec["mfma_counter_frac"] = round(m["mfma_flop"] / (rec["ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    pair = [(MEASURED.get((workload, n, h), {}).get("mfma_flop"), kernels.get(n, {}).get("ms"))
            for n in ("chain_both", "grads")]
    if all(f is not None and t for f, t in pair):
        roof["combined_mfma_counter_frac"] = round(
            sum(f for f, _ in pair) / (sum(t for _, t in pair) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)


def recursion_grid(inp, seq_split: int) -> Dict:
    """The recursions' grid against the CUs (one recursion workgroup fits a CU): the
    reverse role alone can use at most this share of the device (a ceiling on its
    MFMA fraction, whatever its per-CU efficiency).  Unsplit sequences only."""
    H, D = inp["H"], inp["K"]
    segs = len([L for L in inp["lengths"] if L > 0]) if inp["N"] != inp["B"] else inp["B"]
    raw = inp["gate"] == 0 and inp["dtype"] == "bf16"
    # (the launch pads the (sequence, head) pairs to a multiple of 8, one per XCD;
    # two slices a workgroup when the padded grid of both roles exceeds the CUs)
    per_role = ((segs * H + 7) // 8) * 8 * (D // 16)
    nsl = 2 if raw and 2 * per_role > GPU_CUS else 1
    wgs = segs * H * (D // 16) // nsl   # workgroups with work
    rec = {"workgroups_per_role": wgs, "slices_per_workgroup": nsl,
           "reverse_role_cu_share": round(min(1.0, wgs / GPU_CUS), 4)}
    # the library splits sequences (its own choice) only when both roles together
    # leave compute units idle; the figures above are for the unsplit grid
    if seq_split >= 2 or (seq_split == 0 and 2 * H * (D // 16) * segs < GPU_CUS):
        rec["split"] = True
    return rec


def kernel_record(inp, name: str, t: float) -> Dict:
    flops, nbytes = algorithmic_work(inp, name)
    return {"ms": round(t, 4),
            "tflops": round(flops / t / 1e9, 2) if flops else 0.0,
            "mfma_frac": round(flops / t / 1e9 / PEAK_BF16_TFLOPS, 4) if flops else 0.0,
            "gbs": round(nbytes / t / 1e6, 1),
            "hbm_frac": round(nbytes / t / 1e6 / PEAK_HBM_GBS, 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=synth.HEADLINE, choices=synth.WORKLOADS)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--stage-iters", type=int, default=20)
    ap.add_argument("--all-stages", action="store_true",
                    help="also time the forward and reverse recursions alone (two more chain launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy, the reference for HBM byte counters")
    ap.add_argument("--seq-split", type=int, default=0,
                    help="segments per sequence for the two recursions: 0 the library's choice, 1 never split")
    ap.add_argument("--path", choices=("bwd", "fwd"), default="bwd",
                    help="bwd: the backward (gdr_fwd_bwd, the headline); fwd: the forward with its output (gdr_fwd)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU path is not built",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    B.load_library()
    if args.copy_calibration:
        # a plain copy of exactly 1 GiB (read 1 GiB, write 1 GiB): its FETCH_SIZE /
        # WRITE_SIZE counters give the scale for the kernels' counter readings
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    spec = synth.workload(args.workload)
    inp = synth.generate(spec)
    dev = B.to_device(inp)
    prob = B.Problem.from_inputs(inp, seq_split=args.seq_split)
    ws = B.alloc_workspace(prob)
    out = B.alloc_outputs(inp, dev)
    N, H, K, V = inp["N"], inp["H"], inp["K"], inp["V"]
    ht = torch.empty((N, H, V, K), dtype=torch.float32, device="cuda")
    if args.path == "fwd":
        return bench_forward(args, inp, dev, prob, ws, out, ht)

    def step():
        B.gdr_fwd_bwd(prob, dev, dev["dO"], dev["dht"], ws, out, ht=ht)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    times = time_calls(step, args.steps)
    ms = median(times)
    tokens = inp["B"] * inp["T"]

    # every kernel alone (the workspace already holds what earlier stages leave)
    kernels = {}
    # the scalar gate's prepare-backward runs inside its gradient kernel
    # and, with grouped heads, the dq, dk group sums make up the finish stage
    has_finish = inp["gate"] != 0 or (inp.get("Hk") or H) < H
    path = ("prep", "chain_both", "grads") + (("finish",) if has_finish else ())
    stages = [B.GDR_STAGE_PREP, B.GDR_STAGE_CHAIN_BOTH, B.GDR_STAGE_GRADS]
    if has_finish:
        stages.append(B.GDR_STAGE_FINISH)
    if args.all_stages:
        stages += [B.GDR_STAGE_CHAIN_FWD, B.GDR_STAGE_CHAIN_BWD]
    for stage in stages:
        name = B.STAGE_NAMES[stage]
        fn = lambda s=stage: B.gdr_run_stage(prob, dev, dev["dO"], dev["dht"], ws, out, s, ht=ht)  # noqa: E731
        fn()
        kernels[name] = kernel_record(inp, name, median(time_calls(fn, args.stage_iters)))
    dom = max(path, key=lambda n: kernels[n]["ms"])
    roof = roofline(inp, args.workload, dom, kernels[dom]["ms"])
    counters_per_kernel(args.workload, kernels, roof)
    roof["recursion_grid"] = recursion_grid(inp, args.seq_split)

    line = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_mean": round(sum(times) / len(times), 4),
        "timed_region_ms": round(sum(times), 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": inp["B"], "T": inp["T"], "H": H, "Hk": inp.get("Hk") or H, "D": K,
                   "gate": GATE_NAMES[inp["gate"]], "chunk": C, "seq_split": args.seq_split},
        "roofline": roof,
        "path": path_record(inp, ms, path, args.workload),
        "kernels": kernels,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens, inp["T"]))
    print(json.dumps(line), flush=True)
    return 0


def bench_forward(args, inp, dev, prob, ws, out, ht) -> int:
    """The forward with its output (gdr_fwd): prologue, forward state pass, output
    kernel.  The output kernel has no stage of its own: its time is the whole call's
    minus the two stages before it."""
    dt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    o = torch.empty((inp["B"], inp["T"], inp["H"], inp["V"]), dtype=dt, device="cuda")

    def step():
        B.gdr_fwd(prob, dev, ws, o, ht=ht)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    times = time_calls(step, args.steps)
    ms = median(times)
    tokens = inp["B"] * inp["T"]
    kernels = {}
    for stage in (B.GDR_STAGE_PREP, B.GDR_STAGE_CHAIN_FWD):
        name = B.STAGE_NAMES[stage]
        fn = lambda s=stage: B.gdr_run_stage(prob, dev, dev["dO"], dev["dht"], ws, out, s, ht=ht)  # noqa: E731
        fn()
        kernels[name] = kernel_record(inp, name, median(time_calls(fn, args.stage_iters)))
    step()
    t_out = max(median(time_calls(step, args.stage_iters)) - kernels["prep"]["ms"] - kernels["chain_fwd"]["ms"],
                1e-4)
    kernels["output"] = kernel_record(inp, "output", t_out)
    kernels["output"]["derived"] = True
    dom = max(("prep", "chain_fwd"), key=lambda n: kernels[n]["ms"])
    line = {
        "metric": "gated-delta-rule fwd (o, ht) tokens/s + ms/fwd",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_mean": round(sum(times) / len(times), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "path": "fwd", "B": inp["B"], "T": inp["T"], "H": inp["H"],
                   "D": inp["K"], "gate": GATE_NAMES[inp["gate"]], "chunk": C},
        "roofline": roofline(inp, args.workload, dom, kernels[dom]["ms"]),
        "kernels": kernels,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens, inp["T"]), backward=False)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
