"""Benchmark: one step = adaptive solve with record + loss cotangent + replay
discrete-adjoint gradient of a full ensemble (arXiv 2609.02876 Sec. 2.1,
3.1), inputs resident in HBM.

Workload: Lorenz-63, 65,536 trajectories with per-trajectory (sigma, rho,
beta) ~ U[9,11] x U[20,30] x U[2,3], y0 ~ N(0,1)^3 + (1,1,20), t in [0, 2],
Tsit5 rtol 1e-8 atol 1e-10, fp64, loss sum 1/2 |y(2) - target|^2.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload lorenz63]
                    [--no-cpu-baseline]

Prints one JSON line.  `value` = whole-path trajectories/s (solve + gradient);
solves/s and gradient trajectories/s are reported next to it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Algorithmic fp64 flops (fma = 2, add/mul/div/sqrt/pow = 1, compare/abs/neg = 0)
#   per attempted Tsit5 step and per replayed+reversed gradient step.  Derived
#   operation by operation in DESIGN.md ("Algorithmic work").
FLOPS = {
    # system: (flops per solve attempt, flops per gradient step)
    "lorenz63": (255, 606),
}
PEAK_FP64_VALU = 78.6e12  # 256 CU x 4 SIMD x 16 lanes x 2 flop (fma) x 2.4 GHz


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lorenz63")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=65536)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, copy one buffer of MIB MiB once (a plain copy "
                         "kernel of known size, the reference for HBM byte counters)")
    return ap.parse_args()


def cpu_baseline(w, sample):
    """The oracle, as is, on the host cores: solve + gradient of a sample."""
    import numpy as np

    import dao_inputs as di
    import oracle

    nthreads = min(os.cpu_count() or 1, 16)
    ws = di.subset(w, np.arange(min(sample, w.n)))
    t0 = time.perf_counter()
    r = oracle.solve(ws.system, ws.method, ws.theta, ws.y0, ws.t0, ws.t1, ws.rtol, ws.atol,
                     s_cap=2048, nthreads=nthreads)
    lam = di.cotangent(ws, r["y1"])
    oracle.grad(ws.system, ws.method, ws.theta, ws.y0, r["count"], r["h"], lam, nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": ws.n / dt, "unit": "trajectories/s (solve + gradient)", "cores": nthreads,
            "kind": "oracle",
            "sample": f"first {ws.n} of the {w.n} {w.name} trajectories, full solve + tape "
                      f"reverse-mode gradient, {dt:.2f} s wall on {nthreads} threads"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; the ensemble would shard by "
              "trajectory index across GPUs with no exchange (see DESIGN.md). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dao_inputs as di
    import differentiable_adaptive_ode_amd as dao
    from differentiable_adaptive_ode_amd import api

    dev = torch.device("cuda:0")
    w = di.make(args.workload)
    s_cap = {"lorenz63": 1024}[w.name]
    th = torch.tensor(w.theta, device=dev)
    y0 = torch.tensor(w.y0, device=dev)
    tgt = torch.tensor(w.target, device=dev)
    bufs = api.alloc_record(w.n, s_cap, w.dtype, dev, with_t=True)
    y1 = torch.empty_like(y0)
    lam = torch.empty_like(y0)
    dth = torch.empty_like(th)
    dy0 = torch.empty_like(y0)
    wsp = api.Workspace()

    def step(ev):
        ev[0].record()
        rec, _ = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                           out=y1, rec_buffers=bufs, workspace=wsp)
        ev[1].record()
        dao.cotangent(y1, tgt, 1.0, out=lam)
        ev[2].record()
        dao.grad(rec, lam, s_max=s_cap, out_theta=dth, out_y0=dy0, workspace=wsp)
        ev[3].record()
        return rec

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 8, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        rec = step(events())
    torch.cuda.synchronize()

    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        rec = step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_solve = [e[0].elapsed_time(e[1]) * 1e-3 for e in evs]
    t_grad = [e[2].elapsed_time(e[3]) * 1e-3 for e in evs]

    cnt = rec.count.cpu().numpy().astype(np.int64)
    nrej = rec.nrej.cpu().numpy().astype(np.int64)
    status = rec.status.cpu().numpy()
    assert np.all(status == 0), "some trajectories failed"
    attempts = int((cnt + nrej).sum())
    steps_total = int(cnt.sum())
    ms = wall / args.steps * 1e3
    ts, tg = float(np.mean(t_solve)), float(np.mean(t_grad))
    f_att, f_step = FLOPS[w.name]
    fl_solve = attempts * f_att
    fl_grad = steps_total * f_step
    dom = "grad" if tg >= ts else "solve"
    ach = (fl_grad / tg) if dom == "grad" else (fl_solve / ts)
    # Measured HBM bytes per launch of the dominant kernel (rocprofv3 FETCH_SIZE +
    # WRITE_SIZE, copy-calibrated), only if taken on the current kernel sources.
    from differentiable_adaptive_ode_amd.profiling import load_traffic

    tr = load_traffic(w.name)
    traffic = None
    if tr is not None and f"{dom}_kernel" in tr["kernels"]:
        traffic = tr["kernels"][f"{dom}_kernel"]["hbm_bytes"]
    out = {
        "metric": "gradient trajectories/s (replay adjoint) + solves/s at 1 GPU; % of roofline",
        "value": w.n / (wall / args.steps),
        "unit": "trajectories/s (solve with record + replay-adjoint gradient)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"{w.name} ensemble", "n_trajectories": w.n, "method": w.method,
                   "t_span": [w.t0, w.t1], "rtol": w.rtol, "atol": w.atol, "s_cap": s_cap},
        "solves_per_s": w.n / ts,
        "grad_trajectories_per_s": w.n / tg,
        "solve_ms": ts * 1e3,
        "grad_ms": tg * 1e3,
        "accepted_steps_mean": float(cnt.mean()),
        "accepted_steps_max": int(cnt.max()),
        "attempts_total": attempts,
        "solve_fp64_tflops": fl_solve / ts * 1e-12,
        "grad_fp64_tflops": fl_grad / tg * 1e-12,
        "roofline": {"bound": "alu", "kernel": f"{dom}_kernel", "achieved": ach * 1e-12,
                     "peak": PEAK_FP64_VALU * 1e-12, "unit": "TFLOP/s",
                     "frac": ach / PEAK_FP64_VALU, "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch"},
        "roofline_solve_frac": fl_solve / ts / PEAK_FP64_VALU,
        "roofline_grad_frac": fl_grad / tg / PEAK_FP64_VALU,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
