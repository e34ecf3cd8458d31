"""Benchmark of the Dion3 optimizer step on one MI355X.

A step is one call of dion3_step_deferred over the 7B-like transformer shape set
(32 layers x {4 x 4096x4096, 2 x 4096x11008, 1 x 11008x4096}, bf16 W, M, G):
momentum accumulation with l1 keys, top-k selection (k = ceil(f n), f = 1/4 by
default), gather and Frobenius scaling, Gram Newton-Schulz in fp16 (T = 5,
restart after iteration 2) batched over same-shape selected submatrices, and
the fused update of W; the error-feedback decay of the selected lines of M is
applied by the next step's momentum pass (deferred, bit-identical).  Inputs are synthetic and
resident in HBM before the timed region starts; the momentum state carries
across steps.

Prints one JSON line: step milliseconds (the headline, timed with no
per-launch instrumentation), the roofline of the kernel that takes the most
time per step (algorithmic bytes or FLOPs per launch over its average launch
duration, from HIP events recorded around every library launch during a
separate instrumented pass of the same steps), a per-kernel table, the symmetric-GEMM
microbenchmark (C = A A^T and C = A^2 + B on n x n fp16/bf16) and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6    # MI355X dense fp16 / bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X fp32 matrix
MU = 0.95
ETA0 = 0.02                      # eta at f = 1; eta = ETA0 / sqrt(f)


# Single products at the shapes the measurements cite, for rocprofv3 counter
# passes (bench.py --probe NAME): description, and a function that builds the
# operands and returns the launch.
def _probe_syrk(n):
    def make(d, synth, torch):
        A = synth.dense(n, n, 1, dtype="f16", device="cuda:0", seed=1)
        C = torch.empty(1, n, n, dtype=torch.float16, device="cuda:0")
        return lambda: d.dion3_syrk(A, C)
    return make


def _probe_qx(d, synth, torch):
    Q = synth.symmetric(1024, 128, dtype="f16", device="cuda:0", seed=3)
    X = synth.dense(1024, 4096, 128, dtype="f16", device="cuda:0", seed=4)
    Y = torch.empty_like(X)
    return lambda: d.dion3_gemm(Q, X, Y)


def _probe_symmul(d, synth, torch):
    A = synth.symmetric(1024, 128, dtype="f16", device="cuda:0", seed=5)
    B = synth.symmetric(1024, 128, dtype="f16", device="cuda:0", seed=6)
    C = torch.empty_like(A)
    return lambda: d.dion3_sym_mul(A, B, C)


PROBES = {
    "syrk8192": ("C = A A^T, one 8192 x 8192 fp16 A", _probe_syrk(8192)),
    "syrk4096": ("C = A A^T, one 4096 x 4096 fp16 A", _probe_syrk(4096)),
    "qx": ("Y = Q X, 128 x (1024 x 1024 by 1024 x 4096) fp16 (the 7B set's first class at f = 1/4)",
           _probe_qx),
    "symmul": ("C = A B, 128 x 1024 x 1024 symmetric fp16 (the same class's k x k products)", _probe_symmul),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--set", default="7b", choices=["1b", "7b", "14b"])
    ap.add_argument("--f", type=float, default=0.25)
    ap.add_argument("--flavor", default="muon", choices=["muon", "normuon"],
                    help="update flavour (NorMuon: beta2 = 0.95, eps = 1e-8)")
    ap.add_argument("--profile-steps", type=int, default=10,
                    help="steps of the separate instrumented pass that gives the per-kernel table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-microbench", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the step-graph leg")
    ap.add_argument("--probe", choices=list(PROBES), default=None,
                    help="run a few launches of one product and exit (for hardware counters): "
                         + "; ".join(f"{k}: {v[0]}" for k, v in PROBES.items()))
    ap.add_argument("--probe-reps", type=int, default=3)
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size "
                         "reference for hardware byte counters)")
    return ap.parse_args()


# ------------------------------------------------------------------ traffic
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_7b_f025.txt")


def measured_traffic(kernel: str, set_name: str, f: float):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None if there is none for this workload or the
    kernel's source has changed since the counters were taken."""
    import hashlib
    if set_name != "7b" or f != 0.25 or not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        if not line.startswith("traffic "):
            continue
        kv = dict(tok.split("=", 1) for tok in line.split()[1:])
        if kv.get("kernel") != kernel:
            continue
        h = hashlib.sha256()
        for name in (kv["source"], "common.h"):
            with open(os.path.join(ROOT, "muon_momentum_amd", "csrc", name), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest()[:16] != kv["src_sha256"]:
            return None
        return float(kv["total_bytes"])
    return None


# ------------------------------------------------------------ work accounting
def fuses_update(rows, cols, b, k, flavor):
    """Whether the deferred Muon step updates this bf16 group inside its last
    Q X product (row-selected, whole 256 x 256 tiles, at least 128 of them)."""
    m = max(rows, cols)
    return (flavor == "muon" and rows <= cols and k % 256 == 0 and m % 256 == 0
            and b * (k // 256) * (m // 256) >= 128)


def kernel_work(groups, ks, ns_bytes=2, store_bytes=2, flavor="muon"):
    """Algorithmic work per step of every kernel class of the library.

    Bytes: momentum_keys reads M, G and writes M (3 x storage bytes per
    parameter; the deferred decay of the previous selection rides along);
    gather_scale reads each selected element and writes it in the
    Newton-Schulz type; apply_update reads and writes W and reads O per
    selected element (the decay of M is deferred to the next momentum pass).
    FLOPs: a symmetric product counts only its lower triangle (k(k+1)/2
    entries, 2 x contraction length each); Q X is a full k x k by k x m
    product; qx_apply is the last Q X of a group whose update it fuses (that
    group then has no apply_update).  Returns {name: (kind, units per step)}."""
    w = {"momentum_keys": 0.0, "topk_select": 0.0, "gather_scale": 0.0, "apply_update": 0.0,
         "syrk": 0.0, "sym_sq_add": 0.0, "sym_mul": 0.0, "gemm_qx": 0.0, "qx_apply": 0.0,
         "normuon_scale": 0.0}
    for (rows, cols, b), k in zip(groups, ks):
        n, m = min(rows, cols), max(rows, cols)
        fused = fuses_update(rows, cols, b, k, flavor)
        w["momentum_keys"] += b * rows * cols * 3 * store_bytes
        w["topk_select"] += b * n * 8 * 2
        w["gather_scale"] += b * k * m * (store_bytes + ns_bytes)
        if not fused:
            w["apply_update"] += b * k * m * (2 * store_bytes + ns_bytes)
        tri = k * (k + 1) / 2
        last_qx = "qx_apply" if fused else "gemm_qx"
        if k == m:
            # square class: standard Newton-Schulz, per iteration X X^T, A^2 + B, Z X
            w["syrk"] += b * 5 * tri * 2 * m
            w["sym_sq_add"] += b * 5 * tri * 2 * k
            w["gemm_qx"] += b * 4 * 2 * k * k * m
            w[last_qx] += b * 2 * k * k * m
        else:
            passes, iters = 2, 5                     # restart after iteration 2
            w["syrk"] += b * passes * tri * 2 * m
            w["sym_sq_add"] += b * iters * tri * 2 * k
            # Q products: one per iteration except a pass's first (3); Z R Z: two
            # products per iteration except a pass's last (3 iterations -> 6)
            w["sym_mul"] += b * (3 + 6) * tri * 2 * k
            w["gemm_qx"] += b * (passes - 1) * 2 * k * k * m
            w[last_qx] += b * 2 * k * k * m
        # NorMuon flavour: read O once, then the moments and factors
        w["normuon_scale"] += b * k * (m * ns_bytes + 4 * 4)
    kind = {"momentum_keys": "hbm", "topk_select": "hbm", "gather_scale": "hbm",
            "apply_update": "hbm", "syrk": "mfma", "sym_sq_add": "mfma", "sym_mul": "mfma",
            "gemm_qx": "mfma", "qx_apply": "mfma", "normuon_scale": "hbm"}
    return {name: (kind[name], v) for name, v in w.items()}


def cpu_baseline(groups, ks, f, eta, set_name, budget_s=16.0, max_per_group=6):
    """The oracle's whole step on sampled matrices of every shape group (at
    least one each, more while the group's share of `budget_s` lasts); each
    group's time per matrix is scaled by that group's matrix count."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    from muon_momentum_amd import synth

    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    total_s, spent_all, parts = 0.0, 0.0, []
    for gi, ((rows, cols, b), k) in enumerate(zip(groups, ks)):
        spent, done = 0.0, 0
        while done < min(b, max_per_group) and (done == 0 or spent < budget_s / len(groups)):
            W = synth.weights(rows, cols, 1, dtype="bf16", group_seed=1000 + 97 * gi + done)[0]
            G = synth.gradient(rows, cols, 1, dtype="bf16", group_seed=1000 + 97 * gi + done, step=0)[0]
            Wh = W.float().numpy().astype(np.float64)
            Gh = G.float().numpy().astype(np.float64)
            Mh = np.zeros_like(Gh)
            t0 = time.perf_counter()
            O.dion3_step(Wh, Mh, Gh, k=k, mu=MU, eta=eta, fmt="bf16")
            spent += time.perf_counter() - t0
            done += 1
        total_s += spent / done * b
        spent_all += spent
        parts.append(f"{done} of {b} {rows}x{cols}")
    return {"value": round(total_s * 1e3, 1), "unit": "ms per step (extrapolated)",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 NumPy oracle, whole step on {', '.join(parts)} matrices of the {set_name} set "
                       f"at f={f:g} ({spent_all:.1f} s measured); each group's time per matrix scaled by its "
                       f"matrix count")}


# ------------------------------------------------------------- the GPU parts
def run_step_bench(d, synth, torch, args):
    groups = synth.shape_groups(args.set)
    dev = "cuda:0"
    eta = ETA0 / math.sqrt(args.f)
    ks = [d.dion3_k_from_fraction(min(r, c), args.f) for r, c, _ in groups]
    Ws, Ms, Gs, idxs = [], [], [], []
    for gi, (r, c, b) in enumerate(groups):
        Ws.append(synth.weights(r, c, b, dtype="bf16", device=dev, group_seed=gi))
        Gs.append(synth.gradient(r, c, b, dtype="bf16", device=dev, group_seed=gi, step=0))
        Ms.append(torch.zeros(b, r, c, dtype=torch.bfloat16, device=dev))
        idxs.append(torch.empty(b, ks[gi], dtype=torch.int32, device=dev))
    params = d.make_ns_params(ns_dtype=d.F16)
    plan = d.StepPlan(Ws, Ms, Gs, ks, idxs, params)
    torch.cuda.synchronize()
    print(f"# {args.set} set f={args.f:g}: groups {groups} k {ks}; workspace "
          f"{plan.ws.numel() / 2**30:.2f} GiB", file=sys.stderr, flush=True)

    # deferred error feedback: each step's momentum pass applies the decay the
    # previous step's selection owes (bit-identical to decaying in the update)
    Vs = [torch.zeros(b, min(r, c), dtype=torch.float32, device=dev) for r, c, b in groups]

    def one_step(has_prev):
        if args.flavor == "normuon":
            plan.step_normuon(Vs, eta, 0.0, MU, deferred=True, has_prev=has_prev)
        else:
            plan.step_deferred(eta, 0.0, MU, has_prev=has_prev)

    for w in range(args.warmup):
        one_step(w > 0)
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    # host time of one step: the wall time of the call that enqueues it (the
    # queue is drained before each call, so nothing waits on the device)
    host = []
    for _ in range(5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        one_step(True)
        host.append(1e3 * (time.perf_counter() - t0))
    torch.cuda.synchronize()
    host_ms = sorted(host)[len(host) // 2]

    # the headline: K steps with no per-launch instrumentation, one event
    # between consecutive steps (the mean over the timed region and the
    # per-step median / 90th percentile)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        one_step(args.warmup > 0 or i > 0)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    pct = {"p50": per_step[len(per_step) // 2],
           "p90": per_step[min(len(per_step) - 1, int(math.ceil(0.9 * len(per_step))) - 1)]}
    print(f"# timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # the same step as HIP graphs (dion3_step_graph_create, or
    # dion3_step_normuon_graph_create for the NorMuon flavour): per-stream
    # segments replayed on the library's streams ("graph"), and one graph of
    # the whole step ("graph_one"); enqueue time of one launch and K launches
    # timed as above
    if not args.no_graph:
        for key, one in (("graph", False), ("graph_one", True)):
            if args.flavor == "normuon":
                graph = plan.graph_normuon(Vs, eta, 0.0, MU, has_prev=True, one=one)
            else:
                graph = plan.graph(eta, 0.0, MU, has_prev=True, one=one)
            for _ in range(3):
                graph.launch()
            ghost = []
            for _ in range(5):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                graph.launch()
                ghost.append(1e3 * (time.perf_counter() - t0))
            torch.cuda.synchronize()
            ev[0].record()
            for i in range(args.steps):
                graph.launch()
                ev[i + 1].record()
            torch.cuda.synchronize()
            gper = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
            pct[key] = {"ms_per_step": round(ev[0].elapsed_time(ev[-1]) / args.steps, 3),
                        "ms_per_step_p50": round(gper[len(gper) // 2], 3),
                        "host_ms_per_step": round(sorted(ghost)[len(ghost) // 2], 3)}
            graph.destroy()
            torch.cuda.synchronize()
            print(f"# {key} {args.steps} steps: {pct[key]['ms_per_step']:.3f} ms/step", file=sys.stderr,
                  flush=True)

    # a separate instrumented pass for the per-kernel table: a HIP event pair
    # around every library launch, on the stream of the launch
    nprof = max(1, min(args.steps, args.profile_steps))
    launches_per_step = 96
    d.dion3_timing_enable(launches_per_step * nprof + 64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(nprof):
        one_step(True)
    e1.record()
    torch.cuda.synchronize()
    pct["instrumented"] = e0.elapsed_time(e1) / nprof
    pct["profile_steps"] = nprof
    per_kernel = d.dion3_timing_report()
    d.dion3_timing_enable(0)
    print(f"# instrumented {nprof} steps: {pct['instrumented']:.3f} ms/step", file=sys.stderr, flush=True)

    work = kernel_work(groups, ks, flavor=args.flavor)
    table = {}
    for name, (cnt, total_ms) in per_kernel.items():
        kind, units = work.get(name, ("?", 0.0))
        launches = cnt / nprof
        step_ms = total_ms / nprof
        avg_us = 1e3 * total_ms / cnt
        if kind == "hbm":
            ach = units / (step_ms * 1e-3) / 1e9
            peak, unit = HBM_PEAK_GBS, "GB/s"
        else:
            ach = units / (step_ms * 1e-3) / 1e12
            peak, unit = MFMA_F16_PEAK_TFLOPS, "TFLOP/s"
        table[name] = {"launches_per_step": launches, "ms_per_step": round(step_ms, 4),
                       "avg_launch_us": round(avg_us, 2), "bound": kind,
                       "algorithmic_per_launch": units / launches if launches else 0.0,
                       "achieved": round(ach, 2), "unit": unit, "frac": round(ach / peak, 4)}
    del plan, Ws, Ms, Gs, idxs, Vs
    torch.cuda.empty_cache()
    pct["host"] = host_ms
    return ms, pct, table, groups, ks, eta


def run_microbench(d, synth, torch):
    """C = A A^T (n x n A) and C = A^2 + B (symmetric A, B), 10 warm-up and
    50 timed launches each, timed with events on the launching stream."""
    out = []
    for dt in ("f16", "bf16"):
        for n in (2048, 4096, 8192):
            A = synth.dense(n, n, 1, dtype=dt, device="cuda:0", seed=1)
            C = torch.empty(1, n, n, dtype=A.dtype, device="cuda:0")
            S = synth.symmetric(n, 1, dtype=dt, device="cuda:0", seed=1)
            B = synth.symmetric(n, 1, dtype=dt, device="cuda:0", seed=2)
            for op in ("syrk", "sym_sq_add"):
                fn = ((lambda: d.dion3_syrk(A, C)) if op == "syrk"
                      else (lambda: d.dion3_sym_sq_add(S, B, C, 1.0, 1.0, 0.0)))
                for _ in range(10):
                    fn()
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                s.record()
                for _ in range(50):
                    fn()
                e.record()
                torch.cuda.synchronize()
                us = 1e3 * s.elapsed_time(e) / 50
                flop = n * n * (n + 1) + (n * (n + 1) / 2 if op == "sym_sq_add" else 0)
                tf = flop / (us * 1e-6) / 1e12
                out.append({"op": op, "n": n, "dtype": dt, "us": round(us, 2), "tflops": round(tf, 1),
                            "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)})
            del A, C, S, B
    torch.cuda.empty_cache()
    return out


def run_ns_ladder(d, synth, torch, groups, ks):
    """Gram against standard Newton-Schulz (same coefficients, restart after
    iteration 2 for Gram) on one class batch of the workload each: a
    Frobenius-normalised fp16 input of the class's shape [nb][k][m], 2
    warm-up and 5 timed calls of each; ms per call and the ratio."""
    classes = {}
    for (r, c, b), k in zip(groups, ks):
        classes.setdefault((k, max(r, c)), 0)
        classes[(k, max(r, c))] += b
    params = d.make_ns_params(ns_dtype=d.F16)
    out = []
    for (k, m), nb in classes.items():
        if k == m:
            continue
        X = synth.dense(k, m, nb, dtype="f16", device="cuda:0", seed=7, std=1.0 / math.sqrt(k * m))
        O = torch.empty_like(X)
        res = {}
        for name, fn, wsb in (("standard", d.dion3_standard_ns, d.dion3_standard_ns_workspace_bytes),
                              ("gram", d.dion3_gram_ns_gathered, d.dion3_gram_ns_gathered_workspace_bytes)):
            ws = d.workspace(wsb(nb, k, m, d.F16), "cuda:0")
            for _ in range(2):
                fn(X, O, params, ws)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record()
            for _ in range(5):
                fn(X, O, params, ws)
            e.record()
            torch.cuda.synchronize()
            res[name] = s.elapsed_time(e) / 5
            del ws
        out.append({"batch": nb, "k": k, "m": m, "standard_ms": round(res["standard"], 3),
                    "gram_ms": round(res["gram"], 3), "speedup": round(res["standard"] / res["gram"], 2)})
        del X, O
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the step has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import muon_momentum_amd.dion3 as d      # raises if libdion3.so is missing
    from muon_momentum_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.probe:
        fn = PROBES[args.probe][1](d, synth, torch)
        for _ in range(args.probe_reps):
            fn()
        torch.cuda.synchronize()
        print(f"# probe {args.probe} done ({args.probe_reps} launches)", file=sys.stderr, flush=True)
        return

    if args.copy_ref_mib > 0:
        nb = args.copy_ref_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy reference: {args.copy_ref_mib} MiB read + written", file=sys.stderr, flush=True)
        del src, dst

    ms, pct, table, groups, ks, eta = run_step_bench(d, synth, torch, args)
    micro = [] if args.no_microbench else run_microbench(d, synth, torch)
    ladder = [] if args.no_microbench else run_ns_ladder(d, synth, torch, groups, ks)
    if micro:
        print("# microbench done", file=sys.stderr, flush=True)

    dom = max(table, key=lambda k: table[k]["ms_per_step"])
    t = table[dom]
    roof = {"kernel": dom, "bound": t["bound"], "achieved": t["achieved"],
            "peak": HBM_PEAK_GBS if t["bound"] == "hbm" else MFMA_F16_PEAK_TFLOPS,
            "unit": t["unit"], "frac": t["frac"],
            "traffic": measured_traffic(dom, args.set, args.f),
            "avg_launch_us": t["avg_launch_us"]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(groups, ks, args.f, eta, args.set)
        print("# cpu baseline done", file=sys.stderr, flush=True)

    line = {
        "metric": "optimizer step ms (7B shape set, f=1/4) + sym-GEMM TFLOP/s vs MFMA peak",
        "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "ms_per_step_p50": round(pct["p50"], 3), "ms_per_step_p90": round(pct["p90"], 3),
        "host_ms_per_step": round(pct["host"], 3),
        "ms_per_step_instrumented": round(pct["instrumented"], 3),
        "profile_steps": pct["profile_steps"],
        "graph": pct.get("graph"),
        "graph_one": pct.get("graph_one"),
        "data": "synthetic (Gaussian gradients with log-normal line scales, seeded)",
        "config": {"workload": f"{args.set} shape set Dion3 step, f={args.f:g}"
                               + ("" if args.flavor == "muon" else ", NorMuon flavour"),
                   "flavor": args.flavor,
                   "storage": "bf16 W, M, G; f16 Newton-Schulz (fp32 accumulation)",
                   "groups": [list(g) for g in groups], "k": ks, "T": 5, "restart_after": 2,
                   "mu": MU, "eta": eta},
        "roofline": roof,
        "kernels": table,
        "sym_gemm": micro,
        "ns_ladder": ladder,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
