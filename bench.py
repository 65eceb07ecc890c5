#!/usr/bin/env python3
"""Benchmark of the Medusa tree-verify step on one MI355X.

A step is one full pass of the hot path from device-resident decode state:
Medusa heads + top-s + tree fill, embedding, L decoder layers over the tree
(ancestor-masked tree attention, positions n + depth), final norm + LM head,
acceptance with next-root selection, KV compaction.  The timed region replays
the captured step graph `--steps` times with the inputs resident in HBM.

Prints ONE JSON line (rank 0) with steps/s as `value`, tree tokens/s, the
algorithmic HBM bytes per step and the end-to-end fraction of the 8 TB/s
peak, the roofline of the dominant kernel (gate/up GEMM: its launches for
all layers run back to back between HIP events on the library's stream),
and the CPU oracle timed on a bounded sample of the same step on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "tree-verify steps/s + tree tokens/s, 7B-shape 64-node tree, bs1; % HBM peak"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def bytes_model(D, B, T, depth, n_mean, acc_mean):
    """Algorithmic HBM bytes of one step: every weight once (backbone, LM
    head, heads 1..depth), the prefix K/V read once for all T queries, the
    tree's K/V written, the fp32 logits written and read by acceptance, and
    the compaction's row copies."""
    w = 2 * (D.L * (4 * D.d * D.d + 3 * D.d * D.F) + D.V * D.d + depth * (D.d * D.d + D.V * D.d))
    kv = B * D.L * 2 * n_mean * D.d * 2
    tree_kv = B * D.L * 2 * T * D.d * 2
    logits = B * T * D.V * 4 * 2
    compact = B * D.L * 2 * 2 * (1 + acc_mean) * D.d * 2
    return w + kv + tree_kv + logits + compact


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_llama7b_T64_traffic.md")
CSRC = os.path.join(ROOT, "tree_verify_step_amd", "csrc")


# prefill chunk rows (the most the tree-attention kernel takes): 256 rows per
# pass over the weights instead of the tree's 64
PREFILL_ROWS = 256


def gemm_source_hash() -> str:
    """sha256 over the GEMM kernel source, the shared header and the GEMM
    launch table: the counters in the traffic summary hold only while these
    are unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp"):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    api = open(os.path.join(CSRC, "api.cpp")).read()
    m = re.search(r"static GemmCfg gemm_cfg\(.*?\n}\n", api, re.S)
    h.update((m.group(0) if m else "").encode())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, or
    None when it is missing or was taken on a different GEMM source."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = dict(l.split("=", 1) for l in txt.splitlines() if l.startswith(("traffic_", "source_")))
    vals = {k.strip(): v.strip() for k, v in vals.items()}
    if vals.get("source_sha256") != gemm_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_BYTES = 256 << 20          # calibration copy: this many bytes read and written


def calibrate_copy():
    """A plain elementwise copy of known size (float32 negation, 256 MiB in,
    256 MiB out), run three times so that hardware counters taken over the
    program can be scaled to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def pmc_summary(dirs, gate_up_name="gemm_kernel<4, 4, 2, 2>"):
    """Summarise rocprofv3 --pmc counter files (FETCH_SIZE / WRITE_SIZE, KiB
    per dispatch) for the gate/up GEMM, scaled by what the same counter reads
    for the calibration copy."""
    import csv
    import glob
    import statistics
    per = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name, ctr = r["Kernel_Name"], r["Counter_Name"]
                kind = "copy" if "neg" in name else ("gate_up" if gate_up_name in name else None)
                if kind:
                    per.setdefault((kind, ctr), []).append(float(r["Counter_Value"]))
    out = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        cp, gu = per.get(("copy", ctr)), per.get(("gate_up", ctr))
        if not cp or not gu:
            continue
        scale = (COPY_BYTES / 1024) / statistics.median(cp)
        out[ctr] = {"copy_kib": statistics.median(cp), "scale": scale,
                    "gate_up_kib_mean": statistics.mean(gu), "gate_up_dispatches": len(gu),
                    "gate_up_bytes": statistics.mean(gu) * 1024 * scale}
    return out


def gemm_traffic_summary(dirs):
    """Per-kind HBM traffic of the headline step's 64-row GEMM launches from
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes, scaled by what the same
    counter reads for the calibration copy, against each launch's
    algorithmic bytes.  O and down share one instantiation: in dispatch
    order a launch of it after QKV is O, after gate/up down (back-to-back
    timing launches, which follow neither, are left out)."""
    import csv
    import glob
    import statistics
    from workloads import configs
    D, M = configs.HEADLINE.dims, 64
    names = (("QKV", "gemm_kernel<4, 4, 1, 3>"), ("gate/up", "gemm_kernel<4, 4, 2, 2>"),
             ("O / down", "gemm_kernel<4, 4, 1, 1>"), ("LM head", "gemm_kernel<4, 8, 1, 0>"))
    algo = {"QKV": 2 * 3 * D.d * D.d + M * D.d * 2 + M * 3 * D.d * 2,
            "O": 2 * D.d * D.d + M * D.d * (2 + 4 * 2 + 2),
            "gate/up": gate_up_bytes(D, M),
            "down": 2 * D.F * D.d + M * D.F * 2 + M * D.d * (4 * 2 + 2),
            "LM head": 2 * D.V * D.d + M * D.V * 4}
    per, copy = {}, {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Dispatch_Id"]))
            prev = None
            for r in rows:
                name, ctr, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
                if "neg" in name:
                    copy.setdefault(ctr, []).append(v)
                    continue
                kind = next((lab for lab, k in names if k in name), None)
                if kind == "O / down":
                    kind = "O" if prev == "QKV" else "down" if prev == "gate/up" else None
                    prev = None
                elif kind in ("QKV", "gate/up"):
                    prev = kind
                if kind:
                    per.setdefault((kind, ctr), []).append(v)
    lines = []
    for kind in ("QKV", "O", "gate/up", "down", "LM head"):
        tot, parts = 0.0, []
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            vals, cp = per.get((kind, ctr)), copy.get(ctr)
            if not vals or not cp:
                break
            scale = (COPY_BYTES / 1024) / statistics.median(cp)
            b = statistics.mean(vals) * 1024 * scale
            tot += b
            parts.append(f"{ctr} {statistics.mean(vals):.0f} KiB x{scale:.2f} over {len(vals)}")
        else:
            lines.append(f"{kind}: {'; '.join(parts)} -> {tot / 1e6:.2f} MB against "
                         f"{algo[kind] / 1e6:.2f} MB algorithmic ({tot / algo[kind]:.3f}x)")
    return lines


ATTN_KINDS = (("per query block", "tree_attention_qb_kernel"), ("split keys", "tree_attention_kernel<"),
              ("split merge", "attention_merge_kernel"))


def attn_summary(dirs):
    """Summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes for the
    tree-attention kernels (KiB per dispatch), scaled by what the same
    counter reads for the calibration copy."""
    import csv
    import glob
    import statistics
    per = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                name, ctr = r["Kernel_Name"], r["Counter_Name"]
                kind = "copy" if "neg" in name else next((lab for lab, k in ATTN_KINDS if k in name), None)
                if kind:
                    per.setdefault((kind, ctr), []).append(float(r["Counter_Value"]))
    out = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = per.get(("copy", ctr))
        if not cp:
            continue
        scale = (COPY_BYTES / 1024) / statistics.median(cp)
        for lab, _ in ATTN_KINDS:
            v = per.get((lab, ctr))
            if v:
                out[(lab, ctr)] = {"kib_mean": statistics.mean(v), "dispatches": len(v),
                                   "bytes": statistics.mean(v) * 1024 * scale, "scale": scale}
    return out


MFMA_FILE = os.path.join(ROOT, "profiles", "gemm_mfma_llama7b_T64.md")
GEMM_KINDS = (("QKV", "gemm_kernel<4, 4, 1, 3>"), ("O / down", "gemm_kernel<4, 4, 1, 1>"),
              ("gate/up", "gemm_kernel<4, 4, 2, 2>"), ("LM head", "gemm_kernel<4, 8, 1, 0>"))


def mfma_summary(dirs):
    """Summarise a rocprofv3 --pmc MfmaUtil,MfmaFlopsBF16 pass per GEMM kind:
    mean MFMA busy share of all SIMDs while the GPU was busy with the
    dispatch, and bf16 MFMA flops per dispatch."""
    import csv
    import glob
    import statistics
    per = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                for label, name in GEMM_KINDS:
                    if name in r["Kernel_Name"]:
                        per.setdefault((label, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    out = {}
    for label, _ in GEMM_KINDS:
        u, fl = per.get((label, "MfmaUtil")), per.get((label, "MfmaFlopsBF16"))
        if u and fl:
            out[label] = {"util_pct": statistics.mean(u), "flops": statistics.mean(fl),
                          "dispatches": len(u)}
    return out


def recorded_mfma():
    """Gate/up MFMA utilisation from the committed counter summary, or None
    when it is missing or was taken on a different GEMM source."""
    try:
        txt = open(MFMA_FILE).read()
    except OSError:
        return None
    vals = {k.strip(): v.strip() for k, v in
            (l.split("=", 1) for l in txt.splitlines() if l.startswith(("gate_up_", "source_")))}
    if vals.get("source_sha256") != gemm_source_hash():
        return None
    try:
        return {"kernel": "gemm_kernel<4,4,2,EPI_SWIGLU>",
                "util_pct": float(vals["gate_up_mfma_util_pct"]),
                "flops_per_launch": float(vals["gate_up_mfma_flops_per_launch"])}
    except (KeyError, ValueError):
        return None


def gate_up_bytes(D, M):
    """Algorithmic bytes of one gate/up GEMM launch (one layer): gate and up
    weights, the normalised activations in, the SwiGLU output out."""
    return 2 * D.F * D.d * 2 + M * D.d * 2 + M * D.F * 2


def cpu_baseline(w, n0, steps=3, distinct_layers=2):
    """The oracle (float64 NumPy, as it stands) running `steps` whole steps
    of workload `w` for one sequence: all Medusa heads with top-s and tree
    fill, every one of the L decoder layers over the whole tree against an
    n0-token prefix cache (each layer upcasting its float32-held bf16 weights
    to float64, as the oracle does), final norm + LM head, the workload's
    acceptance rule, KV compaction and the next root.  Layer l uses the
    weights of layer l mod `distinct_layers`: the oracle's work does not
    depend on the values, and drawing 32 distinct 7B-sized layers on the host
    would take minutes of input generation."""
    import numpy as np
    from oracle import accept as oa
    from oracle import decode as od
    from oracle import heads as oh
    from oracle import model as om
    from oracle import tree as otree
    from workloads import synth

    D = w.dims
    Wt = synth.Weights(w)

    def get(name):
        if name.startswith("layer"):
            l, rest = name[len("layer"):].split(".", 1)
            name = f"layer{int(l) % distinct_layers}.{rest}"
        return Wt.get(name)

    paths = synth.tree_paths(w, 0)
    t = otree.compile_tree(paths)
    s = synth.tree_topk(w)
    rng = np.random.default_rng(0)
    cap = n0 + steps * (t.max_depth + 1) + t.T
    kv = om.KVCache(D.L, D.H, D.hd, cap)
    for l in range(D.L):
        kv.K[l][:, :n0] = rng.standard_normal((D.H, n0, D.hd))
        kv.V[l][:, :n0] = rng.standard_normal((D.H, n0, D.hd))
    h = rng.standard_normal(D.d)
    t0_tok, n = 1, n0
    # draw the weights up front (input generation is not timed)
    for k in range(1, t.max_depth + 1):
        get(f"head{k}.w1"), get(f"head{k}.w2")
    for l in range(distinct_layers):
        Wt.layer(l)
    get("embed"), get("lm_head"), get("final_norm")
    u = rng.random((steps, t.T))
    t_start = time.perf_counter()
    accepted = 0
    for i in range(steps):
        z = oh.medusa_heads(get, h, t.max_depth)
        tok = otree.fill_tokens(t, t0_tok, oh.head_topk(z, s))
        hn, logits = om.tree_forward(get, D.L, D.H, t, tok, n, kv)
        if w.accept == "greedy":
            res = oa.greedy_accept(t, tok, logits)
        elif w.accept == "typical":
            res = oa.typical_accept(t, tok, logits, w.temperature, w.eps, w.delta)
        else:
            res = oa.reject_accept(t, tok, logits, w.temperature, u[i])
        od.compact_kv(kv, n, res.path)
        n += len(res.path)
        accepted += len(res.path)
        t0_tok = oa.argmax_lowest(logits[res.best])
        h = hn[res.best].copy()
    step = (time.perf_counter() - t_start) / steps
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    return {"value": 1.0 / step, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{steps} whole steps of one sequence: heads and top-s, all {D.L} decoder "
                       f"layers (layer l with layer l mod {distinct_layers}'s weights), final norm "
                       f"and LM head, {w.accept} acceptance, KV compaction; float64 NumPy with "
                       f"the per-layer weight upcast; T={t.T}, n={n0}; {accepted} tokens accepted"),
            "tree_tokens_per_s": t.T / step, "seconds_per_step": step}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_medusa1(D, N=2048, K=4, reps=3):
    """Medusa-1 head training pass (loss and the gradients of W1 and W2) of
    K heads at the workload's width over N positions of seeded bf16 hidden
    states: wall time of the library call between HIP events, and its
    algorithmic bf16 flops over the MFMA peak.  Flops per pass:
    K * 2N (2 d^2 + 3 d V) -- a = H W1^T and dW1 (N d^2 each), z = s W2^T,
    dW2 and ds (N d V each)."""
    import numpy as np
    import torch
    import tree_verify_step_amd as tv
    from tree_verify_step_amd import runtime as rt
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    h = torch.randn(N, D.d, generator=g, device="cuda").to(torch.bfloat16)
    w1 = (torch.randn(K, D.d, D.d, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(K, D.V, D.d, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    labels = torch.randint(0, D.V, (N, K), generator=g, device="cuda", dtype=torch.int32)
    dims = rt.dims_of(D)
    ws = torch.empty(tv.medusa1_workspace_size(dims, N), device="cuda", dtype=torch.uint8)
    loss = torch.zeros(1, device="cuda", dtype=torch.float64)
    dw1 = torch.empty(K, D.d, D.d, device="cuda")
    dw2 = torch.empty(K, D.V, D.d, device="cuda")
    tv.medusa1_loss(dims, N, K, h, labels, None, w1, w2, loss, None, dw1, dw2, ws)   # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        tv.medusa1_loss(dims, N, K, h, labels, None, w1, w2, loss, None, dw1, dw2, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = K * 2.0 * N * (2 * D.d * D.d + 3 * D.d * D.V)
    tflops = flops / (ms * 1e-3) / 1e12
    out = {"positions": N, "heads": K, "width": D.d, "vocab": D.V, "ms": round(ms, 3),
           "tflops": round(tflops, 1), "flops_per_pass": flops,
           "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
           "loss_per_label": round(float(loss.item()) / (N * float(np.sum(0.8 ** np.arange(1, K + 1)))), 4)}
    del ws, dw1, dw2, w1, w2, h
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--profile-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the Medusa-1 head-training pass measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a copy kernel of known size first (for --pmc counter scaling)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc FETCH_SIZE/WRITE_SIZE output dirs and exit")
    ap.add_argument("--mfma-summary", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 output dirs and exit")
    ap.add_argument("--gemm-summary", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc FETCH_SIZE/WRITE_SIZE output dirs for every "
                         "GEMM kind of the headline step and exit")
    ap.add_argument("--attn-summary", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc FETCH_SIZE/WRITE_SIZE output dirs for the "
                         "tree-attention kernels of --workload and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        from workloads import configs
        D = configs.HEADLINE.dims
        res = pmc_summary(args.pmc_summary)
        algo = gate_up_bytes(D, configs.HEADLINE.batch * 64)
        for ctr, v in res.items():
            print(f"{ctr}: copy {v['copy_kib']:.0f} KiB for {COPY_BYTES // 1024} KiB moved "
                  f"(scale {v['scale']:.4f}); gate/up {v['gate_up_kib_mean']:.0f} KiB/dispatch "
                  f"over {v['gate_up_dispatches']} dispatches -> {v['gate_up_bytes'] / 1e6:.2f} MB")
        if "FETCH_SIZE" in res and "WRITE_SIZE" in res:
            tot = res["FETCH_SIZE"]["gate_up_bytes"] + res["WRITE_SIZE"]["gate_up_bytes"]
            print(f"algorithmic_bytes_per_launch = {algo}")
            print(f"traffic_bytes_per_launch = {int(round(tot))}")
            print(f"traffic_over_algorithmic = {tot / algo:.4f}")
            print(f"source_sha256 = {gemm_source_hash()}")
        return 0
    if args.gemm_summary:
        for line in gemm_traffic_summary(args.gemm_summary):
            print(line)
        print(f"source_sha256 = {gemm_source_hash()}")
        return 0
    if args.attn_summary:
        from workloads import configs, synth
        w = configs.get(args.workload) if args.workload else configs.HEADLINE
        D = w.dims
        n = sum(w.prefix) / 2
        T = len(synth.tree_paths(w, 0)) + 1
        # algorithmic bytes of one launch (one layer): the prefix K and V
        # once, the tree's K and V, q read and the output written, bf16
        algo = w.batch * (2 * n * D.d * 2 + 2 * T * D.d * 2 + 2 * T * D.d * 2)
        res = attn_summary(args.attn_summary)
        print(f"workload {w.name}: algorithmic bytes per launch at the initial prefix "
              f"{algo / 1e6:.2f} MB (n = {n:.0f}, T = {T}, batch {w.batch})")
        for (lab, ctr), v in res.items():
            print(f"{lab} {ctr}: {v['kib_mean']:.0f} KiB/dispatch (scale {v['scale']:.4f}) over "
                  f"{v['dispatches']} dispatches -> {v['bytes'] / 1e6:.2f} MB")
        return 0
    if args.mfma_summary:
        from workloads import configs
        D = configs.HEADLINE.dims
        M = configs.HEADLINE.batch * 64
        algo = {"QKV": 2 * M * D.d * 3 * D.d, "O / down": None,
                "gate/up": 2 * M * D.d * 2 * D.F, "LM head": 2 * M * D.d * D.V}
        od = (2 * M * D.d * D.d / 1e9, 2 * M * D.F * D.d / 1e9)
        for label, v in mfma_summary(args.mfma_summary).items():
            a = algo[label]
            print(f"{label}: MFMA busy {v['util_pct']:.2f}% of SIMD cycles, "
                  f"{v['flops'] / 1e9:.3f} GFLOP/dispatch"
                  + (f" (algorithmic {a / 1e9:.3f})" if a else
                     f" (algorithmic: O {od[0]:.3f}, down {od[1]:.3f}; mean {sum(od) / 2:.3f})")
                  + f" over {v['dispatches']} dispatches")
            if label == "gate/up":
                print(f"gate_up_mfma_util_pct = {v['util_pct']:.3f}")
                print(f"gate_up_mfma_flops_per_launch = {v['flops']:.0f}")
        print(f"source_sha256 = {gemm_source_hash()}")
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the tree-verify "
              "step of one sequence batch is a single-GPU workload here", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tree_verify_step_amd as tv
    from tree_verify_step_amd import runtime as rt
    from workloads import configs, synth

    tv.lib()
    if args.calibrate_copy:
        calibrate_copy()
    w = configs.get(args.workload) if args.workload else configs.HEADLINE
    D = w.dims
    B = w.batch
    K, W = args.steps, args.warmup
    P = args.profile_steps if args.profile_steps is not None else K
    s = synth.tree_topk(w)
    paths = [synth.tree_paths(w, b) for b in range(B)]
    ids = synth.prefix_ids(w)
    n0 = [len(x) for x in ids]
    trees = rt.DeviceTrees(paths, s)
    T, depth = trees.T, trees.depth
    chunk = max(T, PREFILL_ROWS)
    cap = ((max(n0) + max(T, chunk) + (K + W + P + 4) * (depth + 1) + 63) // 64) * 64
    log(f"[bench] workload {w.name}: L={D.L} d={D.d} F={D.F} V={D.V} T={T} depth={depth} "
        f"B={B} n0={n0} cap={cap}")
    t_setup = time.perf_counter()
    dw = rt.DeviceWeights(D, None, seed=w.seed_weights, std=w.init_std)
    mode = {"greedy": tv.ACCEPT_GREEDY, "typical": tv.ACCEPT_TYPICAL,
            "reject": tv.ACCEPT_REJECT}[w.accept]
    acc = tv.AcceptParams(mode=mode,
                          root_mode=tv.ROOT_ARGMAX if w.root == "argmax" else tv.ROOT_SAMPLE,
                          temperature=w.temperature, eps=w.eps, delta=w.delta)
    u = synth.uniform_draws(w, K + W + P + 4, T if w.accept == "reject" else 0)
    sess = rt.Session(D, B, T, s, cap, dw, trees, acc, u_draws=u, prefill_rows=chunk)
    sess.prefill(ids)
    torch.cuda.synchronize()
    log(f"[bench] setup + prefill {time.perf_counter() - t_setup:.1f} s")
    # prefill throughput: the prompts again (the first pass loaded the kernels);
    # the library waits for each chunk's host-side counts, so wall time is the
    # device time plus that per-chunk round trip
    t_pf = time.perf_counter()
    sess.prefill(ids)
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - t_pf) * 1e3
    n_chunks = (max(n0) + chunk - 1) // chunk
    prefill = {"prompt_tokens": int(sum(n0)), "chunk_rows": chunk, "chunks": n_chunks,
               "ms": round(prefill_ms, 3), "tokens_per_s": round(sum(n0) / prefill_ms * 1e3, 1)}
    log(f"[bench] prefill of {sum(n0)} tokens in {n_chunks} chunks of {chunk} rows: "
        f"{prefill_ms:.1f} ms ({prefill['tokens_per_s']:.0f} tokens/s)")

    for _ in range(W):
        sess.step(graph=True)
    torch.cuda.synchronize()
    n_start = sess.n_prefix.cpu().numpy().astype(np.int64)
    # events on the library's stream (the default stream) around every step
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    t0 = time.perf_counter()
    for i in range(K):
        sess.step(graph=True)
        evs[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev0, ev1 = evs[0], evs[K]
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(K))
    n_end = sess.n_prefix.cpu().numpy().astype(np.int64)
    wall = t1 - t0
    gpu_ms = ev0.elapsed_time(ev1)
    log(f"[bench] timed {K} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms")
    steps_per_s = K / wall
    ms_per_step = wall * 1e3 / K
    acc_mean = float(np.mean((n_end - n_start) / K - 1))
    n_mean = float(np.mean((n_start + n_end) / 2))
    bstep = bytes_model(D, B, T, depth, n_mean, acc_mean)
    hbm_gbs = bstep * steps_per_s / 1e9

    # per-kind kernel timing: eager steps with HIP events around each launch group
    prof = {}
    for _ in range(P):
        for k, (ms, cnt) in sess.ctx.step_profile().items():
            a = prof.setdefault(k, [0.0, 0])
            a[0] += ms
            a[1] += cnt
    torch.cuda.synchronize()
    kernels = {k: {"ms_per_step": v[0] / P, "avg_launch_us": 1e3 * v[0] / max(v[1], 1),
                   "launches_per_step": v[1] / P} for k, v in prof.items()}
    for k, v in kernels.items():
        log(f"[bench]   {k:14s} {v['ms_per_step']:8.3f} ms/step  {v['avg_launch_us']:8.2f} us/launch"
            f"  x{v['launches_per_step']:.0f}")
    # per-launch durations of the per-layer kernels: each kind's launches for
    # all L layers back to back, HIP events on the library's stream
    for kind in ("gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down", "lm_head"):
        kernels[kind]["isolated_us"] = sess.ctx.time_kernel(kind, reps=3)
        log(f"[bench]   {kind:14s} back-to-back {kernels[kind]['isolated_us']:8.2f} us/launch")
    gu_us = kernels["gemm_gate_up"]["isolated_us"]
    gu_bytes = gate_up_bytes(D, B * T)
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    # the committed counter records describe the 64-row launch of the headline
    # workload; other workloads run other instantiations (wider tiles at more
    # rows), so their lines carry no counter figures
    headline = w.name == configs.HEADLINE.name
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic() if headline else None,
                "kernel": (f"gate/up + SwiGLU GEMM at {B * T} rows, one layer "
                           f"({'gemm_kernel<4,4,2,EPI_SWIGLU>' if B * T <= 64 else 'the launch configuration of that row count'})"),
                "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 2),
                "mfma": recorded_mfma() if headline else None}

    # achievable streaming-read bandwidth of this device (plain read kernel)
    probe = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    read_gbs = (1 << 30) / (tv.read_probe(probe, sink, reps=10) * 1e-6) / 1e9
    del probe
    log(f"[bench] plain streaming read: {read_gbs:.0f} GB/s")

    train = None
    if not args.no_train:
        train = bench_medusa1(D)
        log(f"[bench] Medusa-1 head training pass (N={train['positions']}, K={train['heads']}): "
            f"{train['ms']:.2f} ms, {train['tflops']:.0f} TFLOP/s "
            f"({100 * train['mfma_frac']:.1f}% of the bf16 MFMA peak)")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, n0[0])
        log(f"[bench] oracle: {cpu['seconds_per_step']:.1f} s/step on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init bf16 weights N(0,0.02), uniform random prefix ids, "
                "seeded sparse tree",
        "config": {"workload": w.name, "batch": B, "tree_nodes": T, "tree_depth": depth,
                   "prefix": n0[0] if B == 1 else n0, "acceptance": w.accept,
                   "layers": D.L, "width": D.d, "ffn": D.F, "vocab": D.V, "medusa_heads": D.K},
        "tree_tokens_per_s": round(steps_per_s * B * T, 1),
        "accepted_tokens_per_step": round(1 + acc_mean, 3),
        "hbm_bytes_per_step": int(bstep),
        "hbm_gbs_end_to_end": round(hbm_gbs, 1),
        "hbm_frac_end_to_end": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "read_ceiling_gbs": round(read_gbs, 1),
        "hbm_frac_of_read_ceiling": round(hbm_gbs / read_gbs, 4),
        "graph_event_ms_per_step": round(gpu_ms / K, 4),
        "step_ms_median": round(step_ms[K // 2], 4),
        "step_ms_mean": round(sum(step_ms) / K, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "medusa1_train": train,
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kernels.items()},
    }
    sess.close()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
