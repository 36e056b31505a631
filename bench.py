#!/usr/bin/env python3
"""Benchmark of the AdaFuse pre-gate + one-launch fused merge on one MI355X.

One step = ada_pregate (router GEMV + top-k + gates) -> ada_merge (every layer and
projection, in place, one launch) -> ada_unmerge (one launch), on a seeded synthetic
stack already resident in HBM.  The default workload is the largest that fits one
GPU: the Llama-2-70B-shaped stack (137 GB of bf16 weights, 560 projections) with E=8
adapters of rank 16 per projection and top-2 gating, merged in place.

Prints one JSON line.  `value` is the whole step's algorithmic HBM bytes (W read and
written by merge and by unmerge, the selected adapters read by each, the router read
by pregate) divided by the measured step time.  `roofline` reports the merge kernel
alone: algorithmic bytes per launch over its mean duration from HIP events recorded
on the launch stream inside the timed region.  After the headline stack is freed,
the 7B-shaped stacks (rank 16 top-2, and rank 64 top-4) are timed the same way and
reported under `other_workloads`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
VALU_F32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector peak
METRIC = "full-model adapter merge: effective HBM GB/s (% of peak) and merge µs"
DEFAULT_WORKLOAD = "llama70b_e8r16k2"
DEFAULT_EXTRA = "llama7b_e8r16k2,llama7b_e16r64k4"


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"merge_bf16_traffic_{workload}.txt")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="preset: llama70b_e8r16k2 (default), llama7b_e8r16k2, llama7b_e16r64k4, "
                         "llama70b_tp8_e8r16k2, e2e_llama7b, tiny")
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma-separated presets timed after the headline (merge only, in place); '' for none")
    ap.add_argument("--out-of-place", action="store_true", help="merge into a separate W' buffer")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-copy-ceiling", action="store_true", help="skip timing torch's device copy (torch_copy_GBps)")
    ap.add_argument("--cpu-sample-seconds", type=float, default=10.0,
                    help="oracle time of the CPU baseline's sample (whole layers, at least one)")
    ap.add_argument("--cpu-sample-layers", type=int, default=0, help="cap on the sample's layers (0: none)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="write profiles/merge_bf16_traffic_<workload>.txt from four rocprofv3 --pmc output folders "
                         "(FETCH_SIZE and WRITE_SIZE of this workload's bench run, then of --calibrate-copy "
                         "--calibrate-mib MiB) and exit; needs no GPU")
    ap.add_argument("--calibrate-mib", type=int, default=1024)
    ap.add_argument("--trace-summary", nargs=2, metavar=("DIR", "OUT"),
                    help="write a markdown summary (OUT, under profiles/) of a rocprofv3 --kernel-trace run of this "
                         "command line's workload found under DIR, the timed launches averaged apart from the "
                         "warm-up ones, and exit; needs no GPU")
    ap.add_argument("--trace-command", default="", help="the profiled command, quoted in the trace summary")
    ap.add_argument("--counter-summary", nargs="+", metavar="X",
                    help="OUT DIR [DIR ...]: write a markdown table (OUT, under profiles/) of every counter found "
                         "in the rocprofv3 --pmc output folders DIR, the mean per merge-kernel dispatch, and exit")
    return ap.parse_args()


def _code_only(text: str) -> str:
    """C++ source without comments or blank lines (the merge sources hold no string
    literal containing a comment marker)."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_sha() -> str:
    """Identity of the merge kernel's code (merge.hip and common.h, comments aside):
    a counter summary taken on another code is not reported."""
    h = hashlib.sha256()
    for f in ("merge.hip", "common.h"):
        with open(os.path.join(ROOT, "weight_merge_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, mode: str, path=None):
    """HBM bytes per merge launch from the committed rocprofv3 counter summary, or
    None when the summary is missing or was taken on a different kernel source."""
    path = path or traffic_file(workload)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_sha") != kernel_sha() or rec.get("workload") != workload or rec.get("mode") != mode:
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counter_mean(folder: str, counter: str, kernel_substr: str):
    """Mean per dispatch of one rocprofv3 counter over the kernels whose name contains
    kernel_substr, from the counter_collection.csv files under folder."""
    import csv
    import glob

    total, dispatches, names = 0.0, set(), set()
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if kernel_substr in row["Kernel_Name"] and row["Counter_Name"] == counter:
                    total += float(row["Counter_Value"])
                    dispatches.add(row.get("Dispatch_Id") or row.get("Correlation_Id"))
                    names.add(row["Kernel_Name"])
    if not dispatches:
        raise SystemExit(f"no {counter} samples for '{kernel_substr}' under {folder}")
    return total / len(dispatches), len(dispatches), sorted(names)


def write_traffic(args, cfg, out=None):
    """HBM bytes of one merge launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for torch.neg over a known size."""
    out = out or traffic_file(cfg.name)
    fdir, wdir, cfdir, cwdir = args.traffic_from
    f, nf, names = counter_mean(fdir, "FETCH_SIZE", "merge_bf16_kernel")
    w, nw, _ = counter_mean(wdir, "WRITE_SIZE", "merge_bf16_kernel")
    cf, ncf, _ = counter_mean(cfdir, "FETCH_SIZE", "neg")
    cw, ncw, _ = counter_mean(cwdir, "WRITE_SIZE", "neg")
    cal_kib = args.calibrate_mib * 1024.0
    rf, wf = cal_kib / cf, cal_kib / cw
    rd, wr = f * 1024 * rf, w * 1024 * wf
    alg = cfg.merge_bytes()
    mode = "out_of_place" if args.out_of_place else "in_place"
    flags = (" --workload " + cfg.name if cfg.name != DEFAULT_WORKLOAD else "") + \
        (" --out-of-place" if args.out_of_place else "")
    kname = names[0].replace("void ada::(anonymous namespace)::", "").split("(")[0]
    lines = [
        f"# HBM traffic of one merge launch (rocprofv3 counters), {cfg.name}, {mode.replace('_', ' ')}",
        "#",
        "# Commands (each a pass of its own, run from the repository root on one MI355X):",
        "#   export TMPDIR=/tmp",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fdir} -o p -- python3 bench.py --steps 2 "
        f"--warmup 1 --no-cpu-baseline --no-copy-ceiling --extra ''{flags}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {wdir} -o p -- python3 bench.py --steps 2 "
        f"--warmup 1 --no-cpu-baseline --no-copy-ceiling --extra ''{flags}",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cfdir} -o p -- python3 bench.py "
        f"--calibrate-copy {args.calibrate_mib}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cwdir} -o p -- python3 bench.py "
        f"--calibrate-copy {args.calibrate_mib}",
        f"#   python3 bench.py{flags} --traffic-from {fdir} {wdir} {cfdir} {cwdir} --calibrate-mib {args.calibrate_mib}",
        f"# Counter values are the mean per dispatch of the named kernel ({nf} / {nw} {kname} dispatches: merges "
        f"and unmerges; {ncf} / {ncw} dispatches of torch's neg kernel for the calibration).",
        "#",
        f"# Calibration: torch.neg(a, out=b) on {args.calibrate_mib} MiB bf16 reads and writes exactly "
        f"{cal_kib:.0f} KiB per launch.",
        f"#   FETCH_SIZE read {cf:.1f} KiB -> read factor {rf:.4f}",
        f"#   WRITE_SIZE read {cw:.1f} KiB -> write factor {wf:.4f}",
        f"# Merge kernel: FETCH_SIZE {f:.1f} KiB, WRITE_SIZE {w:.1f} KiB per dispatch",
        f"#   read  = {f:.1f} KiB x 1024 x {rf:.4f} = {rd:.0f} B",
        f"#   write = {w:.1f} KiB x 1024 x {wf:.4f} = {wr:.0f} B",
        f"#   total = {rd + wr:.0f} B per launch; algorithmic bytes {alg} B (ratio {(rd + wr) / alg:.4f})",
        f"kernel_sha: {kernel_sha()}",
        f"workload: {cfg.name}",
        f"mode: {mode}",
        f"read_bytes_per_launch: {rd:.0f}",
        f"write_bytes_per_launch: {wr:.0f}",
        f"traffic_bytes_per_launch: {rd + wr:.0f}",
    ]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}: {rd + wr:.0f} B per launch ({(rd + wr) / alg:.4f} of algorithmic)")


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]


def torch_copy_rate(torch, dev, gib=4.0, reps=10):
    """torch's device-to-device copy of 4 GiB, in GB/s moved (read + write): a
    reference point, not a ceiling (plain 16-byte nontemporal streams run faster)."""
    n = int(gib * (1 << 30)) // 2
    a = torch.empty(n, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * n * 2 / sec / 1e9


def cpu_baseline(cfg, seed, target_s, max_layers=0):
    """The fp64 NumPy oracle on a bounded sample of the same workload: layers 0, 1, ...
    drawn with the same generator as the GPU stack, one step = pregate + merge +
    unmerge, until target_s seconds of oracle time (at least one layer; max_layers
    caps the count when > 0), rated in the benchmark's unit."""
    import numpy as np

    from oracle import adafuse as O
    from weight_merge_amd import synth
    from weight_merge_amd.configs import scaled

    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    limit = cfg.n_layers if max_layers <= 0 else min(max_layers, cfg.n_layers)
    h, R = synth.router_inputs(cfg, seed)
    h64, R64 = h.double().numpy(), R.double().numpy()
    t0 = time.perf_counter()
    idx, g = O.pregate(h64, R64, cfg.k, cfg.renorm)
    sec = time.perf_counter() - t0
    done = 0
    copy_s = 0.0
    while done < limit and (done == 0 or sec < target_s):
        W, A, B = synth.draw_layer(cfg, seed, done, device="cuda")  # layer `done` of the GPU stack
        t0 = time.perf_counter()
        host = [(w.double().cpu().numpy(), a.double().cpu().numpy(), b.double().cpu().numpy())
                for w, a, b in zip(W, A, B)]
        copy_s += time.perf_counter() - t0
        del W, A, B
        t0 = time.perf_counter()
        for Wh, Ah, Bh in host:
            Wm = O.merge(Wh, Ah, Bh, idx, g, cfg.scale)
            O.unmerge(Wm, Ah, Bh, idx, g, cfg.scale)
        sec += time.perf_counter() - t0
        del host
        done += 1
    step_bytes = 2 * scaled(cfg, done).merge_bytes() + (cfg.E * cfg.d_model + cfg.d_model) * cfg.elem_bytes
    return {
        "value": round(step_bytes / sec / 1e9, 3),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"layers 0..{done - 1} of {cfg.n_layers} ({done * len(cfg.projections)} projections, about "
                  f"{target_s:g} s of oracle time): pregate + merge + unmerge in fp64 NumPy, {sec:.2f} s; "
                  f"each layer's inputs copied to host before its timing",
        "seconds": round(sec, 3),
        "device_to_host_copy_seconds": round(copy_s, 3),
        "host": host_description(),
    }


def host_description() -> dict:
    """The host the CPU baseline ran on: CPU model and the BLAS NumPy calls."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy as np

        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "logical_cpus_visible": len(os.sched_getaffinity(0))}


def time_ms(torch, fn, reps):
    """Mean milliseconds of fn() over reps calls, HIP events on the current stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def simple_fusion_ms(torch, st, cfg, idx, gate, reps):
    """The pages' ablation without the fused kernel: one library GEMM per projection,
    W += (s g B_sel) @ A_sel with torch/hipBLASLt (224 launches plus gathers), then the
    same to undo it; returns the mean ms of one such merge."""
    sel = idx.long()
    coef = (cfg.scale * gate).to(torch.bfloat16)

    def merge(sign):
        for l, p, _ in st.items():
            Bs = st.B[l][p].index_select(0, sel) * (sign * coef).view(-1, 1, 1)   # k x d_out x r
            Bcat = Bs.permute(1, 0, 2).reshape(Bs.shape[1], -1)                   # d_out x k r
            Acat = st.A[l][p].index_select(0, sel).reshape(-1, st.A[l][p].shape[2])  # k r x d_in
            st.W[l][p].addmm_(Bcat, Acat)

    for _ in range(2):
        merge(1.0)
        merge(-1.0)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tot = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        e[0].record()
        merge(1.0)
        e[1].record()
        merge(-1.0)
        e[2].record()
        torch.cuda.synchronize()
        tot += e[0].elapsed_time(e[1])
    return tot / reps


def decode_groups(names):
    """Projections of a layer that a decode step can run together: those reading the
    same input.  In a decoder layer q, k and v read the normed hidden state, o reads the
    attention output, gate and up the normed residual, down the activated MLP state."""
    order = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    if sorted(names) == sorted(n for g in order for n in g):
        return [[names.index(n) for n in g] for g in order]
    return [[i] for i in range(len(names))]


def run_e2e(args, cfg, torch, A, synth, dev):
    """End-to-end batch-1 request on the 7B-shaped stack: pregate + merge, decode steps
    through every layer (one GEMV launch per group of projections that read the same
    input), unmerge; against the unmerged per-layer routed baseline (router + base GEMV
    + shrink + expand per projection, every layer, every step), the fused unmerged
    comparator (router + two launches per group), the backbone alone, and a batch of
    requests with mixed selections.  Decode steps are timed eagerly (Python-driven
    launches) and as one captured HIP graph per token."""
    steps = cfg.decode_steps
    st = synth.make_stack(cfg, args.seed, device=dev)
    h, R = synth.router_inputs(cfg, args.seed)
    h, R = h.to(dev), R.to(dev)
    xs = synth.decode_inputs(cfg, args.seed, 1, device=dev)  # one token's activations (content does not change timing)
    x = {name: xs[name][0].contiguous() for name in xs}
    ys = [[torch.empty(proj.d_out, dtype=torch.bfloat16, device=dev) for proj in cfg.projections]
          for _ in range(cfg.n_layers)]
    model = A.AdaModel([(st.W[l][p], None, st.A[l][p], st.B[l][p]) for l, p, _ in st.items()], cfg.E, cfg.r)
    idx = torch.empty(cfg.k, dtype=torch.int32, device=dev)
    gate = torch.empty(cfg.k, dtype=torch.float32, device=dev)
    lidx = [torch.empty(cfg.k, dtype=torch.int32, device=dev) for _ in range(cfg.n_layers)]
    lgate = [torch.empty(cfg.k, dtype=torch.float32, device=dev) for _ in range(cfg.n_layers)]
    ws = [[torch.empty((proj.d_out + cfg.kr + 3) // 4 * 4, dtype=torch.float32, device=dev)
           for proj in cfg.projections] for _ in range(cfg.n_layers)]

    groups = decode_groups([proj.name for proj in cfg.projections])
    names = [proj.name for proj in cfg.projections]

    def token_merged():
        # one launch per group of projections that read the same input
        for l in range(cfg.n_layers):
            for grp in groups:
                A.ada_decode_gemv_layer([(st.W[l][p], x[names[p]], ys[l][p]) for p in grp])

    def token_merged_per_projection():
        for l, p, proj in st.items():
            A.ada_decode_gemv(st.W[l][p], x[proj.name], ys[l][p])

    def token_baseline():
        for l in range(cfg.n_layers):
            A.ada_pregate(h, R, cfg.k, cfg.renorm, lidx[l], lgate[l])
            for p, proj in enumerate(cfg.projections):
                A.ada_lora_apply(st.W[l][p], st.A[l][p], st.B[l][p], lidx[l], lgate[l], cfg.scale, x[proj.name],
                                 ys[l][p], ws[l][p])

    lws = [[torch.empty(A.lora_layer_workspace_elems([cfg.projections[p].d_out for p in grp], cfg.k, cfg.r),
                        dtype=torch.float32, device=dev) for grp in groups] for _ in range(cfg.n_layers)]

    def token_baseline_fused():
        # the strongest unmerged comparator: router + two launches per group of a layer
        for l in range(cfg.n_layers):
            A.ada_pregate(h, R, cfg.k, cfg.renorm, lidx[l], lgate[l])
            for gi, grp in enumerate(groups):
                A.ada_lora_layer([(st.W[l][p], st.A[l][p], st.B[l][p], x[names[p]], ys[l][p]) for p in grp],
                                 lidx[l], lgate[l], cfg.scale, lws[l][gi])

    def graph_of(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    reps = max(3, args.steps)
    # AdaFuse: selection, merge, decode, unmerge
    A.ada_pregate(h, R, cfg.k, cfg.renorm, idx, gate)
    t_pregate = time_ms(torch, lambda: A.ada_pregate(h, R, cfg.k, cfg.renorm, idx, gate), 20)
    pair = time_ms(torch, lambda: (A.ada_merge(model, idx, gate, cfg.scale), A.ada_unmerge(model, idx, gate, cfg.scale)), 5)
    backbone_eager = time_ms(torch, token_merged, reps)      # on unmerged W: the backbone alone
    g_backbone = graph_of(token_merged)
    backbone_graph = time_ms(torch, g_backbone.replay, reps)
    A.ada_merge(model, idx, gate, cfg.scale)
    merged_eager = time_ms(torch, token_merged, reps)
    g_merged = graph_of(token_merged)
    merged_graph = time_ms(torch, g_merged.replay, reps)
    g_merged_pp = graph_of(token_merged_per_projection)
    merged_pp_graph = time_ms(torch, g_merged_pp.replay, reps)
    del g_merged_pp
    A.ada_unmerge(model, idx, gate, cfg.scale)
    # N1: fused in-place switch between two selections (undo prev + apply cur in one pass)
    h2, R2 = synth.router_inputs(cfg, args.seed + 1)
    h2 = h2.to(dev)
    idx2 = torch.empty(cfg.k, dtype=torch.int32, device=dev)
    gate2 = torch.empty(cfg.k, dtype=torch.float32, device=dev)
    A.ada_pregate(h2, R, cfg.k, cfg.renorm, idx2, gate2)
    A.ada_merge(model, idx, gate, cfg.scale)
    sel = [(idx, gate), (idx2, gate2)]
    flip = [0]

    def switch_once():
        a, b = sel[flip[0]], sel[1 - flip[0]]
        A.ada_switch(model, a, b, cfg.scale)
        flip[0] = 1 - flip[0]

    t_switch = time_ms(torch, switch_once, 6)
    if flip[0]:
        switch_once()
    A.ada_unmerge(model, idx, gate, cfg.scale)
    torch.cuda.synchronize()
    # N2: a new selection every decode token, served drift-free: each token is pre-gated
    # on its own hidden state and re-merged from the untouched W into W' (an out-of-place
    # model: one read of W and one write of W' per token, like a switch, and no rounding
    # carried from token to token), then decoded on W'
    wout = [[torch.empty_like(st.W[l][p]) for p in range(len(cfg.projections))] for l in range(cfg.n_layers)]
    model_oop = A.AdaModel([(st.W[l][p], wout[l][p], st.A[l][p], st.B[l][p]) for l, p, _ in st.items()],
                           cfg.E, cfg.r)
    hs = [h, h2]
    tok = [0]

    def token_on_wout():
        for l in range(cfg.n_layers):
            for grp in groups:
                A.ada_decode_gemv_layer([(wout[l][p], x[names[p]], ys[l][p]) for p in grp])

    def token_remerge(ht):
        A.ada_pregate(ht, R, cfg.k, cfg.renorm, idx, gate)
        A.ada_merge(model_oop, idx, gate, cfg.scale)
        token_on_wout()

    def token_remerge_eager():
        token_remerge(hs[tok[0]])
        tok[0] ^= 1

    t_remerge = time_ms(torch, lambda: (A.ada_pregate(h2, R, cfg.k, cfg.renorm, idx, gate),
                                        A.ada_merge(model_oop, idx, gate, cfg.scale)), 6)
    per_token_remerge_eager = time_ms(torch, token_remerge_eager, reps)
    g_re = [graph_of(lambda hh=hh: token_remerge(hh)) for hh in hs]
    rep_i = [0]

    def replay_remerge():
        g_re[rep_i[0]].replay()
        rep_i[0] ^= 1

    per_token_remerge_graph = time_ms(torch, replay_remerge, reps)
    del g_re, model_oop, wout
    torch.cuda.empty_cache()
    base_eager = time_ms(torch, token_baseline, max(2, reps // 4))
    g_base = graph_of(token_baseline)
    base_graph = time_ms(torch, g_base.replay, reps)
    fused_eager = time_ms(torch, token_baseline_fused, max(2, reps // 2))
    g_fused = graph_of(token_baseline_fused)
    fused_graph = time_ms(torch, g_fused.replay, reps)
    del g_backbone, g_merged, g_base, g_fused
    simple = simple_fusion_ms(torch, st, cfg, idx, gate, 3)

    # N4: a batch of requests, each pre-gated once on its own leading token (so each has
    # its own selection), decoding together: a merged backbone holds one selection, so
    # the batch runs the unmerged path, every W row read once per step for all requests
    batch = {}
    for nb in (4, 8, 16):
        bidx = torch.empty(nb, cfg.k, dtype=torch.int32, device=dev)
        bgate = torch.empty(nb, cfg.k, dtype=torch.float32, device=dev)
        for b in range(nb):
            hb, _ = synth.router_inputs(cfg, args.seed + 100 + b)
            A.ada_pregate(hb.to(dev), R, cfg.k, cfg.renorm, bidx[b], bgate[b])
        xb = synth.decode_inputs(cfg, args.seed + 1, nb, device=dev)
        yb = [[torch.empty(nb, proj.d_out, dtype=torch.bfloat16, device=dev) for proj in cfg.projections]
              for _ in range(cfg.n_layers)]
        bws = [[torch.empty(A.lora_batch_workspace_elems([cfg.projections[p].d_out for p in grp], nb, cfg.k,
                                                         cfg.r), dtype=torch.float32, device=dev)
                for grp in groups] for _ in range(cfg.n_layers)]

        def token_batch():
            for l in range(cfg.n_layers):
                for gi, grp in enumerate(groups):
                    A.ada_lora_batch([(st.W[l][p], st.A[l][p], st.B[l][p], xb[names[p]], yb[l][p]) for p in grp],
                                     bidx, bgate, cfg.scale, bws[l][gi])

        g_batch = graph_of(token_batch)
        t_batch = time_ms(torch, g_batch.replay, reps)
        del g_batch
        torch.cuda.synchronize()
        batch[str(nb)] = {
            "distinct_selections": len({tuple(row) for row in bidx.cpu().tolist()}),
            "step_graph_ms": round(t_batch, 4),
            "tokens_per_s": round(nb / t_batch * 1e3, 1),
            "vs_batch1_merged_tokens_per_s": round(nb * merged_graph / t_batch, 3),
            # derived, not timed: serving the same requests one at a time on merged
            # weights, switching the selection before each request's token
            "serial_switching_step_ms_derived": round(nb * (t_remerge + merged_graph), 3),
        }
        del yb, bws, xb

    launches_merged = cfg.n_layers * len(groups)
    launches_base = cfg.n_layers * (1 + 3 * len(cfg.projections))
    req_graph = t_pregate + pair + steps * merged_graph
    req_base_graph = steps * base_graph
    req_eager = t_pregate + pair + steps * merged_eager
    req_base_eager = steps * base_eager
    overhead = t_pregate + pair
    be = None if base_graph <= merged_graph else overhead / (base_graph - merged_graph)
    token_bytes = cfg.decode_bytes_per_token()
    out = {
        "metric": "end-to-end batch-1 request: ms per request and ms per decode token",
        "value": round(req_graph, 3),
        "unit": "ms/request (graph-captured decode)",
        "higher_is_better": False,
        "n_gpus": 1,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,.) draws on the device; no trained weights)",
        "config": {"workload": cfg.note, "preset": cfg.name, "decode_steps": steps, "layers": cfg.n_layers,
                   "E": cfg.E, "r": cfg.r, "k": cfg.k},
        "ms": {
            "pregate": round(t_pregate, 4),
            "merge_plus_unmerge": round(pair, 3),
            "token_backbone_graph": round(backbone_graph, 4),
            "token_merged_graph": round(merged_graph, 4),
            "token_merged_per_projection_graph": round(merged_pp_graph, 4),
            "token_baseline_graph": round(base_graph, 4),
            "token_backbone_eager": round(backbone_eager, 4),
            "token_merged_eager": round(merged_eager, 4),
            "token_baseline_eager": round(base_eager, 4),
            "token_fused_unmerged_graph": round(fused_graph, 4),
            "token_fused_unmerged_eager": round(fused_eager, 4),
            "request_fused_unmerged_graph": round(steps * fused_graph, 3),
            "request_adafuse_graph": round(req_graph, 3),
            "request_baseline_graph": round(req_base_graph, 3),
            "request_adafuse_eager": round(req_eager, 3),
            "request_baseline_eager": round(req_base_eager, 3),
            "simple_fusion_merge": round(simple, 3),
            "switch_in_place": round(t_switch, 3),
            "pregate_plus_remerge": round(t_remerge, 3),
            "token_with_remerge_eager": round(per_token_remerge_eager, 4),
            "token_with_remerge_graph": round(per_token_remerge_graph, 4),
            "request_remerge_every_token_graph": round(steps * per_token_remerge_graph, 3),
        },
        "decode_GBps_merged_graph": round(token_bytes / (merged_graph * 1e-3) / 1e9, 1),
        "launches_per_token": {"merged": launches_merged, "merged_per_projection": cfg.n_layers * len(names),
                               "baseline": launches_base, "fused_unmerged": cfg.n_layers * (1 + 2 * len(groups)),
                               "batch_mixed_selections": cfg.n_layers * 2 * len(groups)},
        "decode_groups": [[names[p] for p in grp] for grp in groups],
        "speedup_request_vs_fused_unmerged_graph": round(steps * fused_graph / req_graph, 3),
        "break_even_tokens_graph": None if be is None else round(be, 1),
        "speedup_request_graph": round(req_base_graph / req_graph, 3),
        "speedup_request_eager": round(req_base_eager / req_eager, 3),
        "overhead_vs_backbone_graph": round(merged_graph / backbone_graph - 1, 4),
        "batch_mixed_selections_unmerged": batch,
    }
    print(json.dumps(out), flush=True)


def kernel_short_name(name: str) -> str:
    return name.replace("void ada::(anonymous namespace)::", "ada::").split("(")[0]


def trace_summary(args, cfg):
    """Markdown summary of a rocprofv3 --kernel-trace run of this workload (default
    flags otherwise): every kernel's calls and mean duration, and the merge kernel's
    launches split into warm-up and timed ones (merge and unmerge alternate, the timed
    ones are the last 2 x steps), with the timed mean's algorithmic GB/s."""
    import csv
    import glob

    folder, out = args.trace_summary
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                rows.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]), row["Kernel_Name"]))
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {folder}")
    rows.sort()
    if cfg.decode_steps:
        return decode_trace_summary(args, cfg, rows, folder, out)
    agent = "gfx950"
    stats = {}
    for t0, t1, name in rows:
        k = kernel_short_name(name)
        c, tot = stats.get(k, (0, 0.0))
        stats[k] = (c + 1, tot + (t1 - t0) / 1e3)
    grand = sum(t for _, t in stats.values())
    merge = [(t0, t1, kernel_short_name(n)) for t0, t1, n in rows if "merge_bf16_kernel" in n or "merge_f32_kernel" in n]
    n_timed = 2 * args.steps
    if len(merge) != 2 * (args.steps + args.warmup):
        raise SystemExit(f"expected {2 * (args.steps + args.warmup)} merge launches, found {len(merge)}: pass the "
                         "profiled run's --steps/--warmup")
    timed = [(t1 - t0) / 1e3 for t0, t1, _ in merge[-n_timed:]]
    warm = [(t1 - t0) / 1e3 for t0, t1, _ in merge[:-n_timed]]
    mean_t = sum(timed) / len(timed)
    alg = cfg.merge_bytes()
    lines = [
        f"# rocprofv3 kernel trace: merge on `{cfg.name}` ({cfg.note})",
        "",
        "Command (from the repository root on one MI355X), and the summary's own command:",
        "",
        "```",
        f"export TMPDIR=/tmp; {args.trace_command}",
        f"python3 bench.py --workload {cfg.name} --steps {args.steps} --warmup {args.warmup} "
        f"--trace-summary {folder} {out}",
        "```",
        "",
        f"Agent: {agent}",
        "",
        "| kernel | calls | total µs | avg µs | % |",
        "|---|---|---|---|---|",
    ]
    for k, (c, tot) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{k[:90]}` | {c} | {tot:.1f} | {tot / c:.2f} | {100 * tot / grand:.1f} |")
    lines += [
        "",
        f"Merge kernel code hash (bench.py kernel_sha, comments aside): {kernel_sha()}.",
        f"Merge kernel launches: {len(merge)} = {args.warmup} warm-up and {args.steps} timed steps, one merge and "
        f"one unmerge each (`{merge[-1][2]}`).",
        f"- warm-up launches: mean {sum(warm) / max(1, len(warm)):.1f} µs over {len(warm)}",
        f"- timed launches: mean {mean_t:.1f} µs, min {min(timed):.1f}, max {max(timed):.1f} over {len(timed)}",
        f"- algorithmic bytes per launch {alg:,} -> {alg / mean_t / 1e3:.0f} GB/s over the timed mean, "
        f"{alg / mean_t / 1e3 / HBM_PEAK_GBPS * 100:.1f}% of {HBM_PEAK_GBPS:.0f} GB/s",
        f"- two timed launches per step: {2 * mean_t / 1e3:.3f} ms of kernel time per step",
    ]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}: timed merge mean {mean_t:.1f} µs ({alg / mean_t / 1e3:.0f} GB/s)")


def decode_trace_summary(args, cfg, rows, folder, out):
    """The end-to-end run's kernel table, and the decode GEMV launches split by group of
    projections: every path launches one gemv_layer_kernel per group, in the order
    {q, k, v}, {o}, {gate, up}, {down}, so the i-th launch belongs to group i mod 4."""
    stats = {}
    for t0, t1, name in rows:
        k = kernel_short_name(name)
        c, tot = stats.get(k, (0, 0.0))
        stats[k] = (c + 1, tot + (t1 - t0) / 1e3)
    grand = sum(t for _, t in stats.values())
    names = [p.name for p in cfg.projections]
    order = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    gbytes = [sum(cfg.projections[names.index(n)].d_out * cfg.projections[names.index(n)].d_in * cfg.elem_bytes
                  for n in g) for g in order]
    gemv = [(t1 - t0) / 1e3 for t0, t1, n in rows if "gemv_layer_kernel" in n]
    lines = [
        f"# rocprofv3 kernel trace: end-to-end request on `{cfg.name}` ({cfg.note})",
        "",
        "Command (from the repository root on one MI355X), and the summary's own command:",
        "",
        "```",
        f"export TMPDIR=/tmp; {args.trace_command}",
        f"python3 bench.py --workload {cfg.name} --steps {args.steps} --trace-summary {folder} {out}",
        "```",
        "",
        "| kernel | calls | total µs | avg µs | % |",
        "|---|---|---|---|---|",
    ]
    for k, (c, tot) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{k[:90]}` | {c} | {tot:.1f} | {tot / c:.2f} | {100 * tot / grand:.1f} |")
    lines += ["", "Decode GEMV launches (`gemv_layer_kernel`) by group of projections (every decode path of the run):",
              "", "| group | launches | bytes per launch | avg µs | GB/s |", "|---|---|---|---|---|"]
    for i, (g, b) in enumerate(zip(order, gbytes)):
        d = gemv[i::4]
        if d:
            m = sum(d) / len(d)
            lines.append(f"| {', '.join(g)} | {len(d)} | {b:,} | {m:.2f} | {b / m / 1e3:.0f} |")
    if gemv:
        per_tok = sum(sum(gemv[i::4]) / max(1, len(gemv[i::4])) for i in range(4)) * cfg.n_layers
        lines.append(f"\nOne token ({cfg.n_layers} layers x 4 launches) at these averages: {per_tok / 1e3:.3f} ms, "
                     f"{cfg.decode_bytes_per_token() / per_tok / 1e3:.0f} GB/s.")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def counter_summary(args, cfg):
    """Markdown table of the rocprofv3 --pmc passes in the given folders: for every
    counter, the mean per dispatch of the merge kernel (summed over the chip)."""
    import csv
    import glob

    out, folders = args.counter_summary[0], args.counter_summary[1:]
    vals, names = {}, set()
    for d in folders:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if "merge_bf16_kernel" not in row["Kernel_Name"] and "merge_f32_kernel" not in row["Kernel_Name"]:
                        continue
                    disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
                    key = (row["Counter_Name"], d)
                    tot = vals.setdefault(key, {})
                    tot[disp] = tot.get(disp, 0.0) + float(row["Counter_Value"])
                    names.add(kernel_short_name(row["Kernel_Name"]))
    if not vals:
        raise SystemExit(f"no merge-kernel counters under {folders}")
    lines = [
        f"# rocprofv3 counters: merge kernel on `{cfg.name}` ({cfg.note})",
        "",
        "Commands (from the repository root on one MI355X; one pass per folder, counters as listed):",
        "",
        "```",
        f"export TMPDIR=/tmp; {args.trace_command}",
        f"python3 bench.py --workload {cfg.name} --counter-summary {' '.join(args.counter_summary)}",
        "```",
        "",
        f"Kernel: {', '.join(f'`{n}`' for n in sorted(names))}; merge kernel code hash (bench.py kernel_sha, comments "
        f"aside): {kernel_sha()}.  Each value is the mean over the pass's merge-kernel dispatches (merges and "
        "unmerges) of the counter summed over the chip.",
        "",
        "| counter | per dispatch | dispatches | pass |",
        "|---|---|---|---|",
    ]
    for (cname, d), per in sorted(vals.items()):
        lines.append(f"| {cname} | {sum(per.values()) / len(per):,.0f} | {len(per)} | `{os.path.basename(d)}` |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}: {len(vals)} counters")


def time_merge_workload(cfg, args, torch, A, synth, dev, steps, warmup, out_of_place):
    """Generate the stack in HBM, then warm-up and timed steps of pregate + merge +
    unmerge; returns the timings (HIP events on the launch stream) and the footprint.
    Frees the stack before returning."""
    torch.cuda.reset_peak_memory_stats(dev)
    t_gen = time.perf_counter()
    st = synth.make_stack(cfg, args.seed, device=dev)
    h, R = synth.router_inputs(cfg, args.seed)
    h, R = h.to(dev), R.to(dev)
    projs = []
    for l, p, _ in st.items():
        w = st.W[l][p]
        projs.append((w, torch.empty_like(w) if out_of_place else None, st.A[l][p], st.B[l][p]))
    model = A.AdaModel(projs, cfg.E, cfg.r)
    idx = torch.empty(cfg.k, dtype=torch.int32, device=dev)
    gate = torch.empty(cfg.k, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    def step(evs=None):
        if evs:
            evs[0].record()
        A.ada_pregate(h, R, cfg.k, cfg.renorm, idx, gate)
        if evs:
            evs[1].record()
        A.ada_merge(model, idx, gate, cfg.scale)
        if evs:
            evs[2].record()
        A.ada_unmerge(model, idx, gate, cfg.scale)
        if evs:
            evs[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print(f"# workload {cfg.name}: {cfg.weight_elems() / 1e9:.2f}G weights, {model.tiles} tiles, "
          f"generated in {gen_s:.1f}s; timing {steps} steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    res = {
        "wall": wall,
        "pre_ms": [e[0].elapsed_time(e[1]) for e in evs],
        "merge_ms": [e[1].elapsed_time(e[2]) for e in evs],
        "unmerge_ms": [e[2].elapsed_time(e[3]) for e in evs],
        "tiles": model.tiles,
        "table_bytes": model.device_bytes,
        "peak_torch_bytes": torch.cuda.max_memory_allocated(dev),
    }
    del model, projs, st, h, R, idx, gate
    torch.cuda.empty_cache()
    return res


def merge_summary(cfg, res, mode):
    merge_ms = res["merge_ms"]
    mean_s = sum(merge_ms) / len(merge_ms) / 1e3
    achieved = cfg.merge_bytes() / mean_s / 1e9
    traffic = read_traffic(cfg.name, mode)
    return mean_s, achieved, traffic


def main():
    args = parse()
    from weight_merge_amd.configs import PRESETS

    if args.traffic_from:
        return write_traffic(args, PRESETS[args.workload])
    if args.trace_summary:
        return trace_summary(args, PRESETS[args.workload])
    if args.counter_summary:
        return counter_summary(args, PRESETS[args.workload])
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the merge needs no communication between GPUs (each merges "
              "its own shard in one launch), so the figure is one MI355X's; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from weight_merge_amd import api as A
    from weight_merge_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        # a plain streaming kernel of known traffic for scaling the HBM byte counters:
        # out-of-place negation reads and writes exactly 2n bytes per launch
        n = args.calibrate_copy * (1 << 20) // 2
        a = torch.ones(n, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"kernel": "neg", "bytes_read_per_launch": 2 * n, "bytes_written_per_launch": 2 * n,
                          "launches": 3}))
        return

    cfg = PRESETS[args.workload]
    if cfg.decode_steps:
        return run_e2e(args, cfg, torch, A, synth, dev)
    mode = "out_of_place" if args.out_of_place else "in_place"
    res = time_merge_workload(cfg, args, torch, A, synth, dev, args.steps, args.warmup, args.out_of_place)

    merge_bytes = cfg.merge_bytes()
    pregate_bytes = (cfg.E * cfg.d_model + cfg.d_model) * cfg.elem_bytes
    step_bytes = 2 * merge_bytes + pregate_bytes
    ms_per_step = res["wall"] * 1e3 / args.steps
    value = step_bytes * args.steps / res["wall"] / 1e9
    merge_mean_s, achieved, traffic = merge_summary(cfg, res, mode)
    merge_ms, unmerge_ms, pre_ms = res["merge_ms"], res["unmerge_ms"], res["pre_ms"]

    torch_copy = None if args.no_copy_ceiling else torch_copy_rate(torch, dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, args.seed, args.cpu_sample_seconds,
                                                          args.cpu_sample_layers)

    others = {}
    for name in [n for n in args.extra.split(",") if n]:
        ocfg = PRESETS[name]
        ores = time_merge_workload(ocfg, args, torch, A, synth, dev, args.steps, args.warmup, False)
        o_mean_s, o_ach, o_traffic = merge_summary(ocfg, ores, "in_place")
        others[name] = {
            "workload": ocfg.note,
            "mode": "in_place",
            "merge_us_mean": round(o_mean_s * 1e6, 1),
            "merge_us_median": round(pct(ores["merge_ms"], 0.5) * 1e3, 1),
            "unmerge_us_median": round(pct(ores["unmerge_ms"], 0.5) * 1e3, 1),
            "merge_algorithmic_bytes": ocfg.merge_bytes(),
            "achieved_GBps": round(o_ach, 2),
            "frac": round(o_ach / HBM_PEAK_GBPS, 4),
            "traffic": None if o_traffic is None else int(o_traffic),
            "target_us_at_70pct": round(ocfg.merge_bytes() / (0.7 * HBM_PEAK_GBPS * 1e3), 1),
            "contraction_frac_of_mfma_peak": round(ocfg.merge_flops() / o_mean_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        }

    wbytes = cfg.weight_elems() * cfg.elem_bytes
    abytes = cfg.adapter_bank_bytes()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,.) draws on the device; no trained weights)",
        "config": {
            "workload": cfg.note,
            "preset": cfg.name,
            "layers": cfg.n_layers,
            "E": cfg.E, "r": cfg.r, "k": cfg.k, "scale": cfg.scale,
            "mode": mode,
            "step": "pregate + merge + unmerge",
            "weights_GB": round(wbytes / 1e9, 3),
            "merge_tiles": res["tiles"],
        },
        "merge_us": {"mean": round(merge_mean_s * 1e6, 1), "median": round(pct(merge_ms, 0.5) * 1e3, 1),
                     "min": round(min(merge_ms) * 1e3, 1), "p90": round(pct(merge_ms, 0.9) * 1e3, 1)},
        "unmerge_us": {"median": round(pct(unmerge_ms, 0.5) * 1e3, 1), "min": round(min(unmerge_ms) * 1e3, 1)},
        "pregate_us": {"median": round(pct(pre_ms, 0.5) * 1e3, 2), "min": round(min(pre_ms) * 1e3, 2)},
        "merge_algorithmic_bytes": merge_bytes,
        "merge_pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "torch_copy_GBps": None if torch_copy is None else round(torch_copy, 1),
        "merge_vs_torch_copy_pct": None if torch_copy is None else round(100 * achieved / torch_copy, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else int(traffic),
            "kernel": "merge_bf16_kernel" if cfg.dtype == "bf16" else "merge_f32_kernel",
            "kernel_sha": kernel_sha(),
        },
        # the rank-k*r product (secondary: the merge is bound by HBM): bf16 runs it on
        # MFMA (dense bf16 peak), fp32 storage on the vector ALUs (fp32 vector peak)
        "contraction": {
            "engine": "mfma" if cfg.dtype == "bf16" else "valu",
            "flops": cfg.merge_flops(),
            "achieved": round(cfg.merge_flops() / merge_mean_s / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else VALU_F32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(cfg.merge_flops() / merge_mean_s / 1e12
                          / (MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else VALU_F32_PEAK_TFLOPS), 4),
        },
        # device footprint beside the base weights: every adapter bank (all E experts of
        # every projection), the merge's work tables, the router and selection
        "memory": {
            "weights_bytes": wbytes,
            "adapter_banks_bytes": abytes,
            "work_table_bytes": res["table_bytes"],
            "peak_device_bytes": res["peak_torch_bytes"] + res["table_bytes"],
            "peak_over_weights": round((res["peak_torch_bytes"] + res["table_bytes"]) / wbytes - 1, 4),
            "out_of_place_copy_bytes": wbytes if args.out_of_place else 0,
        },
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
