#!/usr/bin/env python
"""Benchmark of the Muon group step on one MI355X.

A step here is one pass of the whole hot path over one batch of synthetic
input: fp32 accumulation of the workload's micro-batch gradients, then
muon_step (K1 momentum/norm/copies, grouped Newton-Schulz, K3 scatter).
`value` is the group-step time (muon_step alone, HIP events on the library's
stream, mean over the timed steps); the accumulation is timed beside it.
Inputs are generated on the GPU before the timed region (seeded, Gaussian,
the workload's shapes and sigma).

    python bench.py [--steps K] [--warmup W] [--workload llama7b_32layer]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "Muon group-step time (ms) + NS TFLOP/s as % of bf16 MFMA peak, Llama-7B shapes"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def ns_flops(problems, method: str, steps: int):
    """(nominal, symmetric) Newton-Schulz flops of a group.

    nominal: every product counted in full (standard 20 m^2 n + 10 m^3,
    Gram 4 m^2 n + 34 m^3 at 5 steps).  symmetric: products whose result is
    symmetric (X X^T, A A, and the Gram chain) counted once per output pair,
    which is what the grouped kernel executes (upper-triangle tiles only)."""
    nom = sym = 0.0
    for q in problems:
        m, n = float(q["m"]), float(q["n"])
        if steps == 0:
            continue
        if method == "standard":
            nom += steps * (4 * m * m * n + 2 * m ** 3)
            sym += steps * (3 * m * m * n + m ** 3)
        else:
            chain = steps + (steps - 1) + 2 * (steps - 1)
            nom += 4 * m * m * n + chain * 2 * m ** 3
            sym += 3 * m * m * n + chain * m ** 3
    return nom, sym


def make_inputs(torch, wl, seed: int):
    """Flat device buffers with per-matrix views: micro-batch gradients (two
    buffers, alternated over the micro-batches), the fp32 accumulator (if
    gas > 1), momentum and partitions."""
    dev = torch.device("cuda:0")
    total = wl.numel
    mdt = torch.bfloat16 if wl.micro_dtype == "bf16" else torch.float32
    nbuf = min(wl.gas, 2)
    gen = torch.Generator(device=dev)
    mbs = []
    for b in range(nbuf):
        flat = torch.empty(total, dtype=mdt, device=dev)
        gen.manual_seed(seed + 7919 * b)
        off = 0
        views = []
        for (r, c) in wl.shapes:
            v = flat[off:off + r * c].view(r, c)
            v.copy_(torch.randn((r, c), generator=gen, device=dev, dtype=torch.float32).mul_(wl.sigma))
            views.append(v)
            off += r * c
        mbs.append((flat, views))
    acc = None
    if wl.gas > 1:
        flat = torch.empty(total, dtype=torch.float32, device=dev)
        acc = (flat, _views(flat, wl.shapes))
    mom = torch.zeros(total, dtype=torch.float32, device=dev)
    return mbs, acc, (mom, _views(mom, wl.shapes))


def _views(flat, shapes):
    out, off = [], 0
    for (r, c) in shapes:
        out.append(flat[off:off + r * c].view(r, c))
        off += r * c
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ns_gemm_llama7b_32layer_hbm_traffic.md")
# the sources behind the Llama-7B group's Newton-Schulz launches (all of its
# blocks are 4096 wide, so they run on the large-tile kernel only)
TRAFFIC_SOURCES = ("muon_newton_schulz_step_amd/csrc/k_gemm256.hip", "muon_newton_schulz_step_amd/csrc/plan.cpp",
                   "muon_newton_schulz_step_amd/csrc/tables.hpp", "include/muon.h")


def traffic_sources_hash() -> str:
    """First 16 hex digits of the sha256 of the sources behind the counted
    launches, with comments and whitespace removed (a comment edit does not
    change the kernels the counters were taken on)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, waves: int):
    """HBM bytes per Newton-Schulz launch from the committed FETCH_SIZE /
    WRITE_SIZE summary, or None if it was taken on another workload or wave
    count (a launch covers one wave), or the kernel sources changed since."""
    if workload != "llama7b_32layer" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for ln in open(TRAFFIC_FILE):
        if ":" in ln and not ln.startswith(("|", "#", "`")):
            k, _, v = ln.partition(":")
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256_16") != traffic_sources_hash() or kv.get("waves") != str(waves):
        return None
    try:
        return float(kv["ns_gemm_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, method: str, budget_s: float):
    """The oracle (fp64 numpy, as it stands) on a bounded sample: one matrix
    of each distinct kind (shape and head count) run through the whole step
    (momentum, Newton-Schulz, shape scale, writeback), smallest kinds first,
    while the measured time stays within the budget.  The group time is the
    sum over kinds of count x measured time; kinds left untimed are
    extrapolated by nominal Newton-Schulz flops at the measured rate."""
    import numpy as np
    import oracle.muon_oracle as O
    import workloads as W
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info() if t.get("user_api") == "blas"] or [1])
    except Exception:
        threads = affinity

    def nominal(s, h):
        h = h or 1
        m, n = min(s[0] // h, s[1]), max(s[0] // h, s[1])
        return h * (5 * (4 * m * m * n + 2 * m ** 3) if method == "standard" else 4 * m * m * n + 34 * m ** 3)

    kinds = {}
    for s, h in zip(wl.shapes, wl.heads):
        kinds[(s, h)] = kinds.get((s, h), 0) + 1
    order = sorted(kinds, key=lambda k: nominal(*k))
    probe = O.ns_standard(W.gaussian((512, 512), 1, 1.0).astype(np.float64) / 512.0)  # warm the BLAS
    del probe
    timed, spent, rate = [], 0.0, None
    for (s, h) in order:
        f = nominal(s, h)
        if rate is not None and spent + f / rate > budget_s:
            break
        g = W.gaussian(s, 12345, wl.sigma).astype(np.float64)
        state = O.init_state([s])
        offsets, P = O.pack_layout([s], 1, 16)
        t0 = time.perf_counter()
        O.muon_step([g], state, [s], [h], offsets, 1, P, O.MuonOptions(method=method))
        dt = time.perf_counter() - t0
        spent += dt
        timed.append(((s, h), dt))
        rate = sum(nominal(*k) for k, _ in timed) / spent
        if spent > budget_s:
            break
    done = {k for k, _ in timed}
    total_s = sum(kinds[k] * dt for k, dt in timed) + sum(kinds[k] * nominal(*k) / rate for k in kinds if k not in done)
    desc = ", ".join(f"{s[0]}x{s[1]}{'/%dh' % h if h else ''} ({dt:.2f} s)" for (s, h), dt in timed)
    sampled = sum(kinds[k] for k in done)
    return {"value": round(total_s * 1e3, 1), "unit": "ms", "cores": int(threads), "kind": "oracle",
            "sample": (f"{len(timed)} of the group's {len(wl.shapes)} matrices, one of each kind, through the "
                       f"oracle step (fp64 numpy): {desc}; the group time is count x time per kind" +
                       ("" if len(done) == len(kinds) else ", untimed kinds extrapolated by nominal flops")),
            "extrapolated": sampled != len(timed) or len(done) != len(kinds),
            "timed_s": round(spent, 2), "affinity_cores": int(affinity), "blas_threads": int(threads)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama7b_32layer")
    ap.add_argument("--method", default=None)
    ap.add_argument("--precision", default="bf16")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gram-steps", type=int, default=2,
                    help="timed steps of a second leg in the Gram form when the workload runs both forms and the "
                         "headline is the standard one (0: no Gram leg)")
    ap.add_argument("--max-inflight-gb", type=float, default=None,
                    help="cap the Newton-Schulz workspace at this many GB (the group then runs in waves; default: "
                         "the library's default cap, 24 GiB; 0: no cap)")
    ap.add_argument("--schedule", default="launches", choices=["launches", "persistent"],
                    help="Newton-Schulz schedule of the large-tile blocks: one launch per product, or one "
                         "persistent launch per wave with per-block dependency counters")
    ap.add_argument("--calibrate-copy", type=float, default=0.0,
                    help="only copy this many GiB device-to-device (a plain copy of known size, the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import torch

    import muon_newton_schulz_step_amd as M
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy > 0:
        n = int(args.calibrate_copy * (1 << 30))
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return 0
    M.load()
    wl = W.custom(args.workload) if args.workload.startswith("custom:") else W.ALL[args.workload]()
    method = args.method or wl.methods[0]
    offsets, P = M.pack_layout(wl.shapes, wl.num_partitions, wl.align)
    step_dtype = "fp32" if wl.gas > 1 else wl.micro_dtype
    cap = None if args.max_inflight_gb is None else int(args.max_inflight_gb * 1e9)

    def make_group(meth):
        return M.MuonGroup(wl.shapes, heads=wl.heads, offsets=offsets, num_partitions=wl.num_partitions,
                           partition_numel=P, method=meth, precision=args.precision, grad_dtype=step_dtype,
                           max_inflight_bytes=cap, schedule=args.schedule)

    g = make_group(method)
    log(f"workload {wl.name}: {len(wl.shapes)} matrices, {wl.numel / 1e9:.3f} G elements, method {method}, "
        f"precision {args.precision}, workspace {g.workspace_bytes / 1e9:.1f} GB in {g.stats()['waves']} wave(s)")
    mbs, acc, mom = make_inputs(torch, wl, 1000 * wl.config_id)
    parts_flat = torch.zeros(wl.num_partitions * P, dtype=torch.float32, device="cuda:0")
    parts = [parts_flat[r * P:(r + 1) * P] for r in range(wl.num_partitions)]
    ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device="cuda:0")
    assert ws.data_ptr() % 256 == 0
    torch.cuda.synchronize()
    log("inputs resident")

    def one_step():
        if acc is not None:
            for k in range(wl.gas):
                g.accumulate(acc[1], mbs[k % len(mbs)][1], wl.micro_dtype, k == 0, ws)
            grads = acc[1]
        else:
            grads = mbs[0][1]
        g.step(grads, mom[1], parts, ws)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    g.set_timing(True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    phases, acc_ms = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev0.record()
        if acc is not None:
            for k in range(wl.gas):
                g.accumulate(acc[1], mbs[k % len(mbs)][1], wl.micro_dtype, k == 0, ws)
            grads = acc[1]
        else:
            grads = mbs[0][1]
        ev1.record()
        g.step(grads, mom[1], parts, ws)
        k1, ns, k3, nl = g.phase_ms()
        acc_ms.append(ev0.elapsed_time(ev1))
        phases.append((k1, ns, k3, nl))
        log(f"step {i + 1}/{args.steps}: K1 {k1:.2f} ms, NS {ns:.2f} ms ({nl} launches), K3 {k3:.2f} ms, "
            f"accumulate {acc_ms[-1]:.2f} ms")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the step after the path (update norm, clipping, parameter update on
    # fp32 master partitions), timed on its own after the timed steps
    params_flat = torch.zeros(wl.num_partitions * P, dtype=torch.float32, device="cuda:0")
    params = [params_flat[r * P:(r + 1) * P] for r in range(wl.num_partitions)]
    apply_ms = []
    for i in range(1 + args.steps):
        ev0.record()
        g.apply_update(params, parts, 1e-3, 0.1, 1.0, ws)
        ev1.record()
        torch.cuda.synchronize()
        if i:
            apply_ms.append(ev0.elapsed_time(ev1))
    del params, params_flat

    probs = g.problems()
    nom, sym = ns_flops(probs, method, g.options.ns_steps)
    waves = g.stats()["waves"]
    ws_gb = g.workspace_bytes / 1e9

    # second leg: the same group and inputs in the Gram form (the pages'
    # default method), fewer steps; its own plan and workspace
    gram_leg = None
    if args.gram_steps > 0 and method != "gram" and "gram" in wl.methods:
        g.close()
        del ws
        torch.cuda.empty_cache()
        g = make_group("gram")
        ws = torch.empty(g.workspace_bytes, dtype=torch.uint8, device="cuda:0")
        log(f"Gram leg: workspace {g.workspace_bytes / 1e9:.1f} GB")
        one_step()
        torch.cuda.synchronize()
        g.set_timing(True)
        gp = []
        for i in range(args.gram_steps):
            if acc is not None:
                for k in range(wl.gas):
                    g.accumulate(acc[1], mbs[k % len(mbs)][1], wl.micro_dtype, k == 0, ws)
                grads = acc[1]
            else:
                grads = mbs[0][1]
            g.step(grads, mom[1], parts, ws)
            gp.append(g.phase_ms())
            log(f"Gram step {i + 1}/{args.gram_steps}: K1 {gp[-1][0]:.2f} ms, NS {gp[-1][1]:.2f} ms "
                f"({gp[-1][3]} launches), K3 {gp[-1][2]:.2f} ms")
        torch.cuda.synchronize()
        gnom, gsym = ns_flops(g.problems(), "gram", g.options.ns_steps)
        gk1, gns, gk3 = (statistics.mean(p[j] for p in gp) for j in range(3))
        gram_leg = {"ns_method": "gram", "steps": args.gram_steps, "value": round(gk1 + gns + gk3, 3),
                    "unit": "ms",
                    "phases_ms": {"k1_norm": round(gk1, 3), "newton_schulz": round(gns, 3), "k3_scatter": round(gk3, 3)},
                    "ns_launches": gp[-1][3],
                    "ns_tflops_algorithmic": round(gsym / (gns * 1e-3) / 1e12, 1),
                    "ns_frac_algorithmic": round(gsym / (gns * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "ns_tflops_nominal": round(gnom / (gns * 1e-3) / 1e12, 1),
                    "workspace_gb": round(g.workspace_bytes / 1e9, 1)}
    k1_ms = statistics.mean(p[0] for p in phases)
    ns_ms = statistics.mean(p[1] for p in phases)
    k3_ms = statistics.mean(p[2] for p in phases)
    nl = phases[-1][3]
    group_ms = k1_ms + ns_ms + k3_ms
    numel = wl.numel
    gsz = 4 if step_dtype == "fp32" else 2
    xsz = 2 if args.precision == "bf16" else 4
    k1_bytes = numel * (gsz + 4 + 4 + xsz)          # read G, read m, write m, write X once
    k3_bytes = numel * (xsz + 4)                     # read X_T, write the fp32 partition
    acc_bytes = numel * (2 + 4) + (wl.gas - 1) * numel * (2 + 8) if acc is not None else 0
    peak = PEAK_BF16_TFLOPS if args.precision == "bf16" else PEAK_FP32_TFLOPS
    ns_tflops_sym = sym / (ns_ms * 1e-3) / 1e12
    ns_tflops_nom = nom / (ns_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(group_ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.precision,
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": len(wl.shapes), "numel": numel, "gas": wl.gas,
                   "partitions": wl.num_partitions, "ns_method": method, "ns_steps": g.options.ns_steps,
                   "ns_precision": args.precision, "grad_dtype": step_dtype, "workspace_gb": round(ws_gb, 1),
                   "waves": waves, "ns_schedule": args.schedule},
        "phases_ms": {"k1_norm": round(k1_ms, 3), "newton_schulz": round(ns_ms, 3), "k3_scatter": round(k3_ms, 3),
                      "accumulate": round(statistics.mean(acc_ms), 3) if acc is not None else None,
                      "apply_update": round(statistics.mean(apply_ms), 3)},
        "ns_tflops_nominal": round(ns_tflops_nom, 1),
        "ns_pct_peak_nominal": round(100 * ns_tflops_nom / peak, 2),
        "k1_gbs": round(k1_bytes / (k1_ms * 1e-3) / 1e9, 1),
        "k3_gbs": round(k3_bytes / (k3_ms * 1e-3) / 1e9, 1),
        "accumulate_gbs": round(acc_bytes / (statistics.mean(acc_ms) * 1e-3) / 1e9, 1) if acc is not None else None,
        # read p, read u, write p: 12 B per owned element
        "apply_gbs": round(numel * 12 / (statistics.mean(apply_ms) * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "ns_gemm (grouped Newton-Schulz GEMM)", "bound": "mfma",
                     "achieved": round(ns_tflops_sym, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(ns_tflops_sym / peak, 4), "traffic": measured_traffic(wl.name, waves),
                     "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 FETCH_SIZE/WRITE_SIZE)",
                     "flops_per_step": sym, "launches_per_step": nl,
                     "avg_launch_ms": round(ns_ms / max(nl, 1), 4)},
    }
    if gram_leg is not None:
        line["gram_leg"] = gram_leg
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(wl, method, args.cpu_budget_s)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    g.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
