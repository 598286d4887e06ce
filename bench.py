"""Benchmark: one step = adaptive solve with record + loss cotangent + replay
discrete-adjoint gradient of a full ensemble (arXiv 2609.02876 Sec. 2.1,
3.1), inputs resident in HBM.

Headline workload (the largest benchmark ensemble): 1,048,576 orbits in the
flattened logarithmic halo (arXiv 2609.28458 Sec. 3), per-trajectory (v0, Rc,
q) ~ U[0.9,1.1] x U[0.1,0.3] x U[0.8,1.0], positions ~ N(0,1)^3, velocities
~ N(0,0.5)^3, t in [0, 50], Tsit5 rtol 1e-8 atol 1e-10, fp64, loss on the
final positions.  The line also carries every benchmark ensemble at its own
size (`configs`: Lotka-Volterra 256, Lorenz-63 65,536, the neural field
16,384 in fp32, Robertson 262,144 with Rosenbrock23, the orbits), each with
its solve and gradient times, their fractions of the FP64 vector (or FP32
matrix) peak, algorithmic HBM bytes and the grade against min(peak, AI x HBM
bandwidth), and the oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload loghalo]
                    [--configs 0|1] [--no-cpu-baseline]

Prints one JSON line.  `value` = whole-path trajectories/s (solve + gradient)
of the headline ensemble; solves/s and gradient trajectories/s beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Algorithmic work (flop convention: fma = 2; add, sub, mul, div, sqrt, tanh and
# the controller power = 1; compare, abs, negate, select = 0).
#   init  : f(y0) and the starting step, once per trajectory
#   att   : one attempted step (trial stages, error estimate, test, controller);
#           an accepted step adds one flop (the time update)
#   replay: one replay step (no error estimate), as the gradient's forward pass
# These three are the operation tallies of the oracle's counting scalar on the
# same arithmetic (pinned by tests/test_flop_counts.py).
#   grad  : one accepted step of the gradient = forward replay + recomputed
#           stages + reverse sweep.  Tsit5 (d states, six stage VJPs of V flops
#           each): replay + (replay - 13 d) + 21 + 42 d + 6 V.  Rosenbrock23:
#           replay + (replay - 3 d) + 144 (two transposed solves, two field
#           VJPs, the Jacobian cotangent and its second-derivative pull-back).
#   V per field VJP: Lotka-Volterra 21, Lorenz 19, log halo 41; neural field
#   18954 (W3^T v, W2^T dz2, W1^T dz1, the three weight outer products and the
#   bias sums, tanh derivatives).
def _tsit5_grad(replay, d, v):
    return replay + (replay - 13 * d) + 21 + 42 * d + 6 * v


WORKLOADS = {
    # The record keeps h_n only (the pages: only the step sizes survive the
    # record; t_n is their running sum, which the replay forms itself), 8 bytes
    # per accepted step.  --record-t 1 keeps t_n too.
    # name: s_cap, keep t record, keep the states (the gradient then skips the
    # replay's forward pass; measured slower end to end on every workload here:
    # the solve's extra state writes cost what the replay saves, so off), flops,
    # peak (flop/s), bound, cpu sample size
    "lotka_volterra": dict(s_cap=256, with_t=False, states=False, init=50, att=175, replay=132,
                           grad=_tsit5_grad(132, 2, 21), peak=78.6e12, bound="alu", cpu_n=256),
    "lorenz63": dict(s_cap=1024, with_t=False, states=False, init=68, att=254, replay=192,
                     grad=_tsit5_grad(192, 3, 19), peak=78.6e12, bound="alu", cpu_n=65536),
    "mlp": dict(s_cap=64, with_t=False, states=False, init=18754, att=56337, replay=56256,
                grad=_tsit5_grad(56256, 4, 18954), peak=157.3e12, bound="mfma", cpu_n=1024),
    "robertson": dict(s_cap=1024, with_t=False, states=False, init=68, att=171, replay=105,
                      grad=105 + (105 - 9) + 144, peak=78.6e12, bound="alu", cpu_n=8192),
    "loghalo": dict(s_cap=8192, with_t=False, states=False, init=124, att=497, replay=378,
                    grad=_tsit5_grad(378, 6, 41), peak=78.6e12, bound="alu", cpu_n=2048),
    # the Lorenz ensemble with its difficulty spread (rho log-uniform on
    # [20, 1000]): the same per-unit work, step counts over about 8x
    "lorenz63_spread": dict(s_cap=2048, with_t=False, states=False, init=68, att=254, replay=192,
                            grad=_tsit5_grad(192, 3, 19), peak=78.6e12, bound="alu",
                            cpu_n=8192),
    # HIRES, Rosenbrock23 with the dense 8 x 8 LU of W = I - gamma h J.  Gradient
    # step: replay + stages (replay - 3 d) + reverse 730 = two transposed solves
    # 2 (2 d^2 - d) = 240, the Jacobian cotangent h gamma (rb u^T + F0b k1^T)
    # 4 d^2 = 256, two field VJPs 2 x 76, the Jacobian's pull-back 32, and the
    # cotangent updates 6 d + 2 = 50.
    "hires": dict(s_cap=4096, with_t=False, states=False, init=192, att=1053, replay=807,
                  grad=807 + (807 - 24) + 730, peak=78.6e12, bound="alu", cpu_n=1024),
    # The Verner 7(6) pair on the Lorenz and orbit ensembles.  Not FSAL: an
    # accepted attempt adds one field evaluation (f at the new state; acc_extra
    # = F_f, 8 for Lorenz, 15 for the halo).  Gradient step: replay R + the
    # recomputed stages (R - F_f - 15 d) + the reverse sweep 37 + 76 d + 9 V
    # (seven nonzero weights, nine stage VJPs, thirty nonzero stage couplings).
    "lorenz63_vern7": dict(s_cap=1024, with_t=False, states=False, init=68, att=428,
                           acc_extra=8, replay=321, grad=2 * 321 - 8 - 45 + 37 + 228 + 9 * 19,
                           peak=78.6e12, bound="alu", cpu_n=8192),
    "loghalo_vern7": dict(s_cap=8192, with_t=False, states=False, init=124, att=842,
                          acc_extra=15, replay=633, grad=2 * 633 - 15 - 90 + 37 + 456 + 9 * 41,
                          peak=78.6e12, bound="alu", cpu_n=1024),
    # Rodas5P on the stiff ensembles.  Not FSAL (acc_extra = F_f: Robertson 8,
    # HIRES 35).  Gradient step: replay R + the recomputed stages (R - d) + the
    # reverse 32 d^2 + 93 d + 8 V + 29 + JV: eight transposed solves
    # 8 (2 d^2 - d), the Jacobian cotangent 8 x 2 d^2, eight field VJPs of V
    # flops (Robertson 20, HIRES 76), the 28 C and 15 a stage couplings, the
    # cotangent sums and 1/h, and the Jacobian's pull-back JV (19, 32).
    "robertson_rodas5p": dict(s_cap=1024, with_t=False, states=False, init=68, att=514,
                              acc_extra=8, replay=499,
                              grad=2 * 499 - 3 + 32 * 9 + 93 * 3 + 8 * 20 + 29 + 19,
                              peak=78.6e12, bound="alu", cpu_n=8192),
    "hires_rodas5p": dict(s_cap=2048, with_t=False, states=False, init=192, att=2356,
                          acc_extra=35, replay=2338,
                          grad=2 * 2338 - 8 + 32 * 64 + 93 * 8 + 8 * 76 + 29 + 32,
                          peak=78.6e12, bound="alu", cpu_n=1024),
}
# Forward sensitivities (solve_sens, Tsit5): per accepted step and parameter
# direction, the stage tangents and the tangent update take 48 d flops, plus
# six field JVPs; JVP_SUM is one JVP's flops summed over the p parameter
# directions (decay 2, Lotka-Volterra 4 x 15, Lorenz 15 + 14 + 13, Robertson
# 14 + 15 + 15, log halo 34 + 36 + 35).
JVP_SUM = {"decay": 2, "lotka_volterra": 60, "lorenz63": 42, "robertson": 44, "loghalo": 105}
# Rosenbrock23's tangent per direction: two Jacobian-tangent products with the
# stages (2 d^2 + 2 d, 2 d^2 + 3 d), two solves with the step's LU factors
# (2 d^2 - d each), 5 d vector updates = 8 d^2 + 8 d; plus two field JVPs and
# one Jacobian JVP (JJVP_SUM over the p directions: decay 0, Lotka-Volterra
# 4 x 14, Lorenz 3 x 1, Robertson 3 x 11).
JJVP_SUM = {"decay": 0, "lotka_volterra": 56, "lorenz63": 3, "robertson": 33}


def _sens_step_flops(d, p, name, method):
    if method == "rosenbrock23":
        return p * (8 * d * d + 8 * d) + 2 * JVP_SUM[name] + JJVP_SUM[name]
    return 48 * d * p + 6 * JVP_SUM[name]


# MI355X published peaks: FP64 vector 78.6 TFLOP/s (256 CU x 4 SIMD x 16 lanes x
# 2 flop x 2.4 GHz); FP32 matrix (MFMA) 157.3 TFLOP/s.


# The pages' own speed-ups, quoted as context only: other hardware, other
# libraries and other workloads, so no ratio to this line is formed
# (vs_baseline stays null).
PAGES_CONTEXT = {
    "forward": "2.8x over DiffEqGPU.jl's fused GPUTsit5 kernel (gradsolve, the forward-only "
               "kernel's comparison: A100-SXM4, fp64, Tsit5, an ensemble of 1.05e6)",
    "gradient": "5.6-14.1x over Diffrax's checkpointed adjoint (gradsolve Figure 8: A100, H100, "
                "RTX 4090, Lorenz ensemble-size sweep)",
    "note": "NVIDIA hardware and other codes: context, not a target",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="loghalo", choices=sorted(WORKLOADS),
                    help="the headline ensemble (default: the largest, the log-halo orbits)")
    ap.add_argument("--n", type=int, default=None,
                    help="trajectories (default: the workload's own ensemble size); e.g. the "
                         "Lotka-Volterra system at n = 1048576, where its 256-trajectory "
                         "ensemble cannot fill the chip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--configs", type=int, choices=(0, 1), default=1,
                    help="gradient mode: also measure every benchmark ensemble at its own size "
                         "(the per-config block of the line)")
    ap.add_argument("--config-steps", type=int, default=10,
                    help="timed steps of each other ensemble in the per-config block")
    ap.add_argument("--mode", choices=("gradient", "sens", "replay_sens", "states", "grad_at"),
                    default="gradient",
                    help="gradient: solve with record + replay-adjoint gradient (default); "
                         "sens: solve with the forward sensitivities dy1/dtheta in the same "
                         "kernel; replay_sens: dy1/dtheta by forward mode through the replay "
                         "of a record; states: the states at 16 requested times on a record; "
                         "grad_at: the gradient of a loss on the states at 16 requested times "
                         "and at t1, on a record")
    ap.add_argument("--states", action="store_true",
                    help="record states in the solve; the gradient skips the forward replay")
    ap.add_argument("--record-t", type=int, choices=(0, 1), default=None,
                    help="keep t_n in the record beside h_n (default: the workload's setting)")
    ap.add_argument("--graph", type=int, choices=(0, 1), default=1,
                    help="gradient mode: also time the step replayed as one captured HIP graph "
                         "(the same launches without per-launch host overhead); value and "
                         "ms_per_step then come from the replays, the per-kernel figures from "
                         "the eager steps")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="trajectories in the CPU-baseline sample (default per workload)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, copy one buffer of MIB MiB once (a plain copy "
                         "kernel of known size, the reference for HBM byte counters)")
    return ap.parse_args()


def _issued(tr, kern, fl_alg, f64):
    """Issued floating-point work of one call of `kern` (its one or two
    launches) from the profile's instruction counters, when they were taken on
    the current kernel sources and ensemble size, and the vector units'
    utilisation = algorithmic flops / issued flops (padding steps and masked
    lanes are issued but are no work of the method)."""
    if tr is None:
        return None
    for key in (kern, kern.replace("_kernel", "_phased_kernel")):
        iss = tr["kernels"].get(key, {}).get("issued")
        if iss:
            tot = (iss["fp64_lane_flops"] if f64
                   else iss["mfma_f32_flops"] + (iss.get("counter_flops_fp32") or 0.0))
            if tot > 0:
                return {"issued_flops": tot, "utilisation": fl_alg / tot}
    return None


def _divergence(cnt, nrej, attempts, steps_total, t_solve, t_grad):
    import numpy as np

    def lockstep(x):
        pad = (-len(x)) % 64
        g = np.concatenate([x, np.zeros(pad, x.dtype)]).reshape(-1, 64)
        return float(g.max(axis=1).sum() * 64 / max(x.sum(), 1))

    att = cnt + nrej
    return {"attempts_per_s": attempts / t_solve, "replay_steps_per_s": steps_total / t_grad,
            "attempts_p50_p99_max": [int(np.percentile(att, 50)), int(np.percentile(att, 99)),
                                     int(att.max())],
            "lockstep_factor_solve": lockstep(att),
            "lockstep_factor_grad_sorted": lockstep(np.sort(cnt)[::-1].copy())}


def copy_calibration(mib, dev):
    """One device-to-device copy of a known size: the reference that scales the
    HBM byte counters of a profiled run."""
    import torch

    if mib > 0:
        src = torch.ones((mib << 20) // 8, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


# The five benchmark ensembles, in order (Lotka-Volterra 256; Lorenz-63 65,536;
# the neural field 16,384 in binary32; Robertson 262,144 with Rosenbrock23;
# the log-halo orbits 1,048,576).  The headline is the largest, the orbits.
CONFIGS = ["lotka_volterra", "lorenz63", "mlp", "robertson", "loghalo"]
HBM_PEAK = 8.0e12  # bytes/s, MI355X HBM3E (published)
# oracle samples per workload: (solve, gradient, one-thread) trajectories
CPU_SAMPLES = {"lotka_volterra": (256, 256, 256), "lorenz63": (65536, 32768, 1024),
               "mlp": (16384, 4096, 128), "robertson": (131072, 32768, 1024),
               "loghalo": (16384, 4096, 64), "hires": (8192, 2048, 64),
               "lorenz63_spread": (32768, 8192, 512), "lorenz63_vern7": (65536, 32768, 1024),
               "loghalo_vern7": (16384, 4096, 64), "robertson_rodas5p": (131072, 32768, 1024),
               "hires_rodas5p": (8192, 2048, 64)}


def cpu_threads():
    """Host threads the oracle baseline runs on: the threads this process may
    use, at most 16 (the host CPU share of one GPU on an 8-GPU node)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(avail, 16))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, s_cap, n_solve, n_grad, n_single):
    """The oracle, as is, on the host cores: its solve with record and its
    tape reverse-mode gradient timed separately on samples of the ensemble
    (the gradient on the sample's own oracle mesh) on the machine's CPU share, and
    both again on one thread for the time per trajectory."""
    import numpy as np

    import dao_inputs as di
    import oracle

    T = cpu_threads()

    def run(n, threads, grad=True):
        ws = di.subset(w, np.arange(min(n, w.n)))
        t0 = time.perf_counter()
        r = oracle.solve(ws.system, ws.method, ws.theta, ws.y0, ws.t0, ws.t1, ws.rtol, ws.atol,
                         s_cap=s_cap, dtype=ws.dtype, nthreads=threads)
        ts = time.perf_counter() - t0
        tg = None
        if grad:
            lam = di.cotangent(ws, r["y1"].astype(np.float64))
            t0 = time.perf_counter()
            oracle.grad(ws.system, ws.method, ws.theta.astype(np.float64),
                        ws.y0.astype(np.float64), r["count"], r["h"].astype(np.float64), lam,
                        nthreads=threads)
            tg = time.perf_counter() - t0
        return ws.n, ts, tg

    ns, ts, _ = run(n_solve, T, grad=False)
    ng, _, tg = run(n_grad, T)
    n1, ts1, tg1 = run(n_single, 1)
    solve_rate, grad_rate = ns / ts, ng / tg
    return {"value": 1.0 / (1.0 / solve_rate + 1.0 / grad_rate),
            "unit": "trajectories/s (solve with record + replay-adjoint gradient)",
            "cores": T, "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "solves_per_s": solve_rate, "grad_trajectories_per_s": grad_rate,
            "single_thread_us_per_trajectory": {"solve": ts1 / n1 * 1e6, "grad": tg1 / n1 * 1e6},
            "sample": (f"{w.name}: solve of the first {ns} of {w.n} trajectories "
                       f"({ts:.2f} s), tape gradient of the first {ng} on their oracle mesh "
                       f"({tg:.2f} s), {T} threads; one thread: {n1} trajectories")}


def solve_bytes(w, steps_total, with_t):
    """Algorithmic HBM bytes of one solve call: parameters and initial states
    read, final states, counts and statuses written, one record row (h, and
    t when kept) per accepted step."""
    r = 8 if w.dtype == "f64" else 4
    p = w.theta.shape[0]
    th = p * r if w.system == "mlp" else p * r * w.n
    return th + w.n * (2 * w.d * r + 12) + steps_total * r * (2 if with_t else 1)


def grad_bytes(w, steps_total, rows):
    """Algorithmic HBM bytes of one ordered gradient call: per trajectory the
    parameters, initial state, cotangent, count, status and order read and the
    two gradients written; per accepted step h read once and the stored state
    written and read back (with the step's h: d + 1 values each way); the
    neural field keeps d values per step and adds the rows of partial weight
    gradients (one per chunk of 16-trajectory groups), written and read by the
    reduction."""
    r = 8 if w.dtype == "f64" else 4
    p = w.theta.shape[0]
    if w.system == "mlp":
        per_traj = 3 * w.d * r + 12
        return (p * r + w.n * per_traj + steps_total * (r + 2 * w.d * r)
                + rows * p * r * 2 + p * r)
    per_traj = (2 * p + 3 * w.d) * r + 12
    return w.n * per_traj + steps_total * (r + 2 * (w.d + 1) * r)


def measure_gradient(w, args, steps, warmup, graph):
    """One step = solve with record + loss cotangent + sort + replay-adjoint
    gradient, timed `steps` times after `warmup` (and, with graph, replayed as
    one captured HIP graph).  Returns the workload's measurement record."""
    import numpy as np
    import torch

    import differentiable_adaptive_ode_amd as dao
    from differentiable_adaptive_ode_amd import api

    dev = torch.device("cuda:0")
    cfg = WORKLOADS[w.name]
    s_cap = cfg["s_cap"]
    th = torch.tensor(w.theta, device=dev)
    y0 = torch.tensor(w.y0, device=dev)
    tgt = torch.tensor(w.target, device=dev)
    states = cfg["states"] or args.states
    with_t = cfg["with_t"] if args.record_t is None else bool(args.record_t)
    bufs = api.alloc_record(w.n, s_cap, w.dtype, dev, with_t=with_t,
                            states_dim=w.d if states else 0)
    # cotangent of the workload's loss: 1/2 |y - target|^2 (positions only for
    # the orbits), or the mean square over the n x d entries (neural field)
    d_used = 3 if w.loss == "half_sq_pos" else w.d
    scale = 2.0 / (w.n * w.d) if w.loss == "mse" else 1.0
    y1 = torch.empty_like(y0)
    lam = torch.empty_like(y0)
    dth = torch.empty_like(th)
    dy0 = torch.empty_like(y0)
    wsp = api.Workspace()
    s_max = [s_cap]

    # One step: solve with record | loss cotangent | order the trajectories by
    # step count | gradient kernel.  The library launches on torch's current
    # stream, so torch's events on that stream bracket each part.
    def step(ev):
        ev[0].record()
        rec, _ = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                           out=y1, rec_buffers=bufs, workspace=wsp)
        ev[1].record()
        dao.cotangent(y1, tgt, scale, d_used=d_used, out=lam)
        ev[2].record()
        dao.grad_order(rec, s_max=s_max[0], workspace=wsp)
        ev[3].record()
        dao.grad(rec, lam, s_max=s_max[0], out_theta=dth, out_y0=dy0, workspace=wsp, ordered=True)
        ev[4].record()
        return rec

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    copy_calibration(args.copy_calibration, dev)

    # The record's longest row sizes the gradient's checkpoint scratch.  Every
    # step solves the same inputs, so it is read once, after the first solve
    # (the record summary, read back before the timed steps).
    rec = step(events())
    s_max[0] = rec.stats_host()["s_max"]
    for _ in range(max(warmup - 1, 0)):
        rec = step(events())
    torch.cuda.synchronize()

    evs = [events() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        rec = step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_solve = [e[0].elapsed_time(e[1]) * 1e-3 for e in evs]
    t_grad = [e[2].elapsed_time(e[4]) * 1e-3 for e in evs]
    t_kern = [e[3].elapsed_time(e[4]) * 1e-3 for e in evs]

    # The same step captured once as a HIP graph and replayed: identical launches
    # on the same buffers, without the host's per-launch overhead.  Every
    # replay must reproduce the eager step's outputs.
    ms_eager = wall / steps * 1e3
    launch = "eager"
    graph_note = None
    if graph:
        class _NoEvent:
            def record(self):
                pass

        noev = [_NoEvent()] * 5
        ref = (dth.clone(), dy0.clone(), y1.clone())

        def same():
            # Every output is bit-reproducible, the neural field's
            # shared-weight sum included (its partial sums are per chunk of
            # groups in a stable order, summed in a fixed order).
            return (torch.equal(dth, ref[0]) and torch.equal(dy0, ref[1])
                    and torch.equal(y1, ref[2]))

        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(noev)
            torch.cuda.synchronize()
            for _ in range(max(warmup, 1)):
                g.replay()
            torch.cuda.synchronize()
            if not same():
                raise RuntimeError("a graph replay differs from the eager step")
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            wall_graph = time.perf_counter() - t0
            if not same():
                raise RuntimeError("a graph replay differs from the eager step")
            wall = wall_graph  # only once every replay checked out
            launch = "hip graph"
        except Exception as e:  # report the eager timing instead
            graph_note = f"graph replay not used: {e}"

    cnt = rec.count.cpu().numpy().astype(np.int64)
    nrej = rec.nrej.cpu().numpy().astype(np.int64)
    status = rec.status.cpu().numpy()
    if not np.all(status == 0):
        bad = np.bincount(status, minlength=5)
        raise SystemExit(f"bench: some trajectories failed (status counts {bad.tolist()})")
    attempts = int((cnt + nrej).sum())
    steps_total = int(cnt.sum())
    ts, tg, tk = float(np.mean(t_solve)), float(np.mean(t_grad)), float(np.mean(t_kern))
    fl_solve = (w.n * cfg["init"] + attempts * cfg["att"]
                + steps_total * (1 + cfg.get("acc_extra", 0)))
    # with recorded states the gradient does no forward replay
    fl_grad = steps_total * (cfg["grad"] - (cfg["replay"] if states else 0))
    peak = cfg["peak"]
    rows = min(-(-w.n // 16), 2048)  # the neural gradient's partial-sum rows (chunks)
    by_solve = solve_bytes(w, steps_total, with_t)
    by_grad = grad_bytes(w, steps_total, rows)

    def part(fl, by, t):
        # graded against the attainable rate min(peak, AI x HBM bandwidth)
        ai = fl / by
        attain = min(peak, ai * HBM_PEAK)
        return {"ms": t * 1e3, "alg_flops": fl, "tflops": fl / t * 1e-12,
                "frac_peak": fl / t / peak, "alg_bytes": by, "alg_hbm_gbps": by / t * 1e-9,
                "hbm_frac": by / t / HBM_PEAK, "arith_intensity": ai,
                "bound": "hbm" if ai * HBM_PEAK < peak else cfg["bound"],
                "attainable_tflops": attain * 1e-12, "graded_frac": fl / t / attain}

    # Measured HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    # copy-calibrated), only if taken on the current kernel sources.
    from differentiable_adaptive_ode_amd.profiling import load_traffic

    tr = load_traffic(w.name, w.n)
    psolve, pgrad = part(fl_solve, by_solve, ts), part(fl_grad, by_grad, tk)
    for kind, pk in (("solve", psolve), ("grad", pgrad)):
        pk["measured_hbm_bytes"] = None
        for key in (f"{kind}_kernel", f"{kind}_phased_kernel"):  # one or two launches
            if tr is not None and pk["measured_hbm_bytes"] is None and key in tr["kernels"]:
                pk["measured_hbm_bytes"] = tr["kernels"][key]["hbm_bytes"]
    out = {
        "workload": f"{w.name} ensemble", "n_trajectories": w.n, "method": w.method,
        "dtype": w.dtype, "t_span": [w.t0, w.t1], "rtol": w.rtol, "atol": w.atol,
        "s_cap": s_cap, "s_max": s_max[0], "recorded_states": states, "record_t": with_t,
        "ms_per_step": wall / steps * 1e3, "launch": launch, "ms_per_step_eager": ms_eager,
        "launch_note": graph_note, "steps": steps, "warmup": warmup,
        "trajectories_per_s": w.n / (wall / steps),
        "solves_per_s": w.n / ts, "grad_trajectories_per_s": w.n / tg,
        "solve_ms": ts * 1e3, "grad_ms": tg * 1e3, "grad_kernel_ms": tk * 1e3,
        "grad_order_ms": (tg - tk) * 1e3,
        "accepted_steps_mean": float(cnt.mean()), "accepted_steps_max": int(cnt.max()),
        "attempts_total": attempts,
        # divergence: the work rate per lane-attempt, and what a lockstep code
        # would issue instead (groups of 64 consecutive trajectories for the
        # solve, each group running as long as its longest member; the
        # gradient's groups are sorted by step count first)
        "divergence": _divergence(cnt, nrej, attempts, steps_total, ts, tk),
        "solve": psolve, "grad": pgrad, "peak_tflops": peak * 1e-12, "peak_kind": cfg["bound"],
        # issued vs algorithmic flops per call (profile counters), or null
        "issue": {"solve": _issued(tr, "solve_kernel", fl_solve, w.dtype == "f64"),
                  "grad": _issued(tr, "grad_kernel", fl_grad, w.dtype == "f64")},
    }
    del bufs, wsp, th, y0, tgt, y1, lam, dth, dy0, rec
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def roofline_of(m):
    """The bench line's roofline object: the dominant kernel of the step (the
    solve call or the ordered gradient call), graded against its own bound:
    FP64 vector (or FP32 matrix) flops at or above the ridge AI = peak / HBM
    bandwidth, HBM bytes below it."""
    dom = "grad" if m["grad_kernel_ms"] >= m["solve_ms"] else "solve"
    p = m[dom]
    if p["bound"] == "hbm":
        ach, peak, unit = p["alg_hbm_gbps"], HBM_PEAK * 1e-9, "GB/s"
    else:
        ach, peak, unit = p["tflops"], m["peak_tflops"], "TFLOP/s"
    return {"bound": p["bound"], "kernel": f"{dom}_kernel", "launch_ms": p["ms"],
            "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
            "traffic": p["measured_hbm_bytes"],
            "traffic_unit": "HBM bytes per call (two launches for a two-phase solve)",
            "alg_bytes": p["alg_bytes"], "arith_intensity": p["arith_intensity"],
            "graded_frac": p["graded_frac"]}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on exactly one GPU; the ensemble would shard by "
              "trajectory index across GPUs, with no exchange for per-trajectory parameters "
              "and one all-reduce of the shared weights otherwise. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import dao_inputs as di

    w = di.make(args.workload, args.n)
    if args.mode in ("sens", "replay_sens") and w.name not in JVP_SUM:
        # HIRES is differentiated with respect to its initial state (its rate
        # constants are fixed), so its forward sensitivities are not benchmarked
        raise SystemExit(f"bench: no forward-sensitivity benchmark for {w.name}")
    if args.mode == "sens":
        return bench_sens(args, w)
    if args.mode in ("replay_sens", "states", "grad_at"):
        return bench_on_record(args, w)

    head = measure_gradient(w, args, args.steps, args.warmup, bool(args.graph))
    print(f"bench: {w.name} n={w.n} measured ({head['ms_per_step']:.3f} ms/step)",
          file=sys.stderr, flush=True)
    out = {
        "metric": "gradient trajectories/s (replay adjoint) + solves/s at 1 GPU; % of roofline",
        "value": head["trajectories_per_s"],
        "unit": "trajectories/s (solve with record + replay-adjoint gradient)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "launch": head["launch"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": head["workload"], "n_trajectories": w.n, "method": w.method,
                   "t_span": [w.t0, w.t1], "rtol": w.rtol, "atol": w.atol,
                   "s_cap": head["s_cap"]},
        "solves_per_s": head["solves_per_s"],
        "grad_trajectories_per_s": head["grad_trajectories_per_s"],
        "solve_ms": head["solve_ms"], "grad_ms": head["grad_ms"],
        "roofline": roofline_of(head),
        "roofline_solve_frac": head["solve"]["frac_peak"],
        "roofline_grad_frac": head["grad"]["frac_peak"],
        "headline": head,
        "context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        samp = CPU_SAMPLES[w.name] if args.cpu_sample is None else (args.cpu_sample,) * 3
        out["cpu_baseline"] = cpu_baseline(w, WORKLOADS[w.name]["s_cap"], *samp)
        print("bench: cpu baseline done", file=sys.stderr, flush=True)
    if args.configs and args.n is None:
        # every benchmark ensemble at its own size: the same step and figures
        per = {}
        for name in CONFIGS:
            wc = w if name == w.name else di.make(name)
            m = head if name == w.name else measure_gradient(wc, args, args.config_steps,
                                                             args.warmup, bool(args.graph))
            rec = {k: m[k] for k in ("n_trajectories", "method", "dtype", "ms_per_step",
                                      "launch", "trajectories_per_s", "solves_per_s",
                                      "grad_trajectories_per_s", "solve_ms", "grad_ms",
                                      "grad_kernel_ms", "accepted_steps_mean",
                                      "accepted_steps_max", "solve", "grad", "issue")}
            rec["roofline"] = roofline_of(m)
            if not args.no_cpu_baseline:
                rec["cpu_baseline"] = (out["cpu_baseline"] if name == w.name else
                                       cpu_baseline(wc, WORKLOADS[name]["s_cap"],
                                                    *CPU_SAMPLES[name]))
            per[name] = rec
            print(f"bench: config {name} done ({m['ms_per_step']:.3f} ms/step)", file=sys.stderr,
                  flush=True)
        out["configs"] = per
    print(json.dumps(out), flush=True)


def cpu_baseline_sens(w, sample, s_cap):
    """The oracle, as is: solve + dual-number forward sensitivities of a sample."""
    import numpy as np

    import dao_inputs as di
    import oracle

    nthreads = min(os.cpu_count() or 1, 16)
    ws = di.subset(w, np.arange(min(sample, w.n)))
    t0 = time.perf_counter()
    r = oracle.solve(ws.system, ws.method, ws.theta, ws.y0, ws.t0, ws.t1, ws.rtol, ws.atol,
                     s_cap=s_cap, dtype=ws.dtype, nthreads=nthreads)
    oracle.sens(ws.system, ws.method, ws.theta, ws.y0, r["count"], r["h"], with_y0=False,
                nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": ws.n / dt, "unit": "trajectories/s (solve + forward sensitivities)",
            "cores": nthreads, "kind": "oracle",
            "sample": f"first {ws.n} of the {w.n} {w.name} trajectories, full solve + dual-number "
                      f"forward sensitivities on its mesh, {dt:.2f} s wall on {nthreads} threads"}


def bench_sens(args, w):
    """One step = dao_solve_sens: the adaptive solve with record and the forward
    sensitivities S = dy1/dtheta integrated in the same kernel (application
    paper arXiv 2609.28458 Sec. 2.3, Sec. 3)."""
    import numpy as np
    import torch

    import differentiable_adaptive_ode_amd as dao
    from differentiable_adaptive_ode_amd import api

    dev = torch.device("cuda:0")
    cfg = WORKLOADS[w.name]
    s_cap = cfg["s_cap"]
    th = torch.tensor(w.theta, device=dev)
    y0 = torch.tensor(w.y0, device=dev)
    bufs = api.alloc_record(w.n, s_cap, w.dtype, dev, with_t=cfg["with_t"])
    y1 = torch.empty_like(y0)
    S = torch.empty((w.d, w.theta.shape[0], w.n), dtype=y0.dtype, device=dev)
    wsp = api.Workspace()

    def run(ev, sens):
        ev[0].record()
        if sens:
            dao.solve_sens(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                           out=y1, rec_buffers=bufs, workspace=wsp, out_sens=S)
        else:
            dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                      out=y1, rec_buffers=bufs, workspace=wsp)
        ev[1].record()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    copy_calibration(args.copy_calibration, dev)
    for _ in range(max(args.warmup, 1)):
        run(events(), True)
        run(events(), False)
    torch.cuda.synchronize()
    plain = [events() for _ in range(args.steps)]
    for e in plain:
        run(e, False)
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        run(e, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tk = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    tp = float(np.mean([e[0].elapsed_time(e[1]) for e in plain])) * 1e-3
    cnt = bufs["count"].cpu().numpy().astype(np.int64)
    nrej = bufs["nrej"].cpu().numpy().astype(np.int64)
    if not np.all(bufs["status"].cpu().numpy() == 0):
        raise SystemExit("bench: some trajectories failed")
    attempts, steps_total = int((cnt + nrej).sum()), int(cnt.sum())
    fl_solve = w.n * cfg["init"] + attempts * cfg["att"] + steps_total
    fl_sens = steps_total * _sens_step_flops(w.d, w.theta.shape[0], w.name, w.method)
    ach = (fl_solve + fl_sens) / tk
    from differentiable_adaptive_ode_amd.profiling import load_traffic

    tr = load_traffic(f"{w.name}_sens", w.n)
    kern = "solve_sens_kernel"
    traffic = None
    for key in ("solve_sens_kernel", "solve_sens_phased_kernel"):  # one or two launches
        if tr and traffic is None and key in tr["kernels"]:
            traffic = tr["kernels"][key]["hbm_bytes"]
    out = {
        "metric": "forward-sensitivity trajectories/s (solve + dy1/dtheta in one kernel) at 1 GPU",
        "value": w.n / (wall / args.steps),
        "unit": "trajectories/s (solve with record + forward sensitivities)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} ensemble, forward sensitivities", "n_trajectories": w.n,
                   "method": w.method, "t_span": [w.t0, w.t1], "rtol": w.rtol, "atol": w.atol,
                   "s_cap": s_cap, "directions": int(w.theta.shape[0])},
        "solve_sens_ms": tk * 1e3, "solve_ms": tp * 1e3,
        "accepted_steps_mean": float(cnt.mean()), "attempts_total": attempts,
        "roofline": {"bound": cfg["bound"], "kernel": "solve_sens_kernel",
                     "launch_ms": tk * 1e3, "achieved": ach * 1e-12, "peak": cfg["peak"] * 1e-12,
                     "unit": "TFLOP/s", "frac": ach / cfg["peak"], "traffic": traffic,
                     "traffic_unit": "HBM bytes per call (two launches for a two-phase solve)"},
        "issue": _issued(tr, "solve_sens_kernel", fl_solve + fl_sens, w.dtype == "f64"),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_sens(w, args.cpu_sample or min(cfg["cpu_n"], 4096),
                                                s_cap)
    print(json.dumps(out), flush=True)


STATES_M = 16  # requested times of the states benchmark, uniform over [t0, t1]


def cpu_baseline_on_record(w, sample, s_cap, mode):
    """The oracle, as is: forward mode through the replay, or the states at the
    requested times, on a sample's own mesh (the solve is setup, not timed)."""
    import numpy as np

    import dao_inputs as di
    import oracle

    nthreads = min(os.cpu_count() or 1, 16)
    ws = di.subset(w, np.arange(min(sample, w.n)))
    r = oracle.solve(ws.system, ws.method, ws.theta, ws.y0, ws.t0, ws.t1, ws.rtol, ws.atol,
                     s_cap=s_cap, dtype=ws.dtype, nthreads=nthreads)
    t0 = time.perf_counter()
    if mode == "replay_sens":
        oracle.sens(ws.system, ws.method, ws.theta, ws.y0, r["count"], r["h"], with_y0=False,
                    nthreads=nthreads)
        what = "dual-number forward sensitivities through the replay of its mesh"
    elif mode == "grad_at":
        tq = np.linspace(ws.t0, ws.t1, STATES_M)
        rng = np.random.default_rng(0)
        cq = rng.normal(size=(STATES_M,) + ws.y0.shape)
        oracle.grad_at(ws.system, ws.method, ws.theta, ws.y0, ws.t0, ws.t1, r["count"], r["h"],
                       tq, cq, dLdy1=rng.normal(size=ws.y0.shape), nthreads=nthreads)
        what = (f"tape gradient of a loss on the states at {STATES_M} requested times and t1, "
                "on its mesh")
    else:
        tq = np.linspace(ws.t0, ws.t1, STATES_M)
        oracle.states_at(ws.system, ws.method, ws.theta, ws.y0, ws.t0, ws.t1, r["count"], r["h"],
                         tq, nthreads=nthreads)
        what = f"states at {STATES_M} requested times on its mesh"
    dt = time.perf_counter() - t0
    return {"value": ws.n / dt, "unit": "trajectories/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {ws.n} of the {w.n} {w.name} trajectories, {what} (the oracle's "
                      f"solve of the sample is setup), {dt:.2f} s wall on {nthreads} threads"}


def bench_on_record(args, w):
    """One step on a recorded mesh (the solve that writes it is setup, untimed):
    replay_sens = dao_sens, dy1/dtheta by forward mode through the replay
    (application paper arXiv 2609.28458 Sec. 2.3; gradsolve Sec. 3.1);
    states = dao_states_at at STATES_M requested times, a shortened step from
    the start of the step holding each (application paper Appendix A)."""
    import numpy as np
    import torch

    import differentiable_adaptive_ode_amd as dao
    from differentiable_adaptive_ode_amd import api

    if w.name == "mlp":
        raise SystemExit("bench: forward sensitivities and states at requested times are "
                         "provided for the per-trajectory systems, not the neural field")
    dev = torch.device("cuda:0")
    cfg = WORKLOADS[w.name]
    s_cap = cfg["s_cap"]
    th = torch.tensor(w.theta, device=dev)
    y0 = torch.tensor(w.y0, device=dev)
    wsp = api.Workspace()
    rec, _ = dao.solve(w.system, w.method, th, y0, w.t0, w.t1, w.rtol, w.atol, s_cap=s_cap,
                       record_t=cfg["with_t"], workspace=wsp)
    torch.cuda.synchronize()
    cnt = rec.count.cpu().numpy().astype(np.int64)
    if not np.all(rec.status.cpu().numpy() == 0):
        raise SystemExit("bench: some trajectories failed")
    s_max = int(cnt.max())
    steps_total = int(cnt.sum())
    tq = torch.linspace(w.t0, w.t1, STATES_M, dtype=y0.dtype, device=dev)
    yq = torch.empty((STATES_M, w.d, w.n), dtype=y0.dtype, device=dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    cq = torch.randn((STATES_M, w.d, w.n), dtype=y0.dtype, device=dev, generator=gen)
    c1 = torch.randn((w.d, w.n), dtype=y0.dtype, device=dev, generator=gen)
    dth = torch.empty_like(th)
    dy0 = torch.empty_like(y0)

    def run(ev):
        ev[0].record()
        if args.mode == "replay_sens":
            dao.sens(rec, s_max=s_max, workspace=wsp)
        elif args.mode == "grad_at":
            dao.grad_at(rec, tq, cq, c1, s_max=s_max, out_theta=dth, out_y0=dy0, workspace=wsp)
        else:
            dao.states_at(rec, tq, s_max=s_max, out=yq, workspace=wsp)
        ev[1].record()

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    copy_calibration(args.copy_calibration, dev)
    for _ in range(max(args.warmup, 1)):
        run(events())
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tk = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    p = int(w.theta.shape[0])
    if args.mode == "replay_sens":
        # per accepted step: the replay step and the tangent along p directions
        fl = steps_total * (cfg["replay"] + _sens_step_flops(w.d, p, w.name, w.method))
        kern, label, tag = "sens_kernel", "forward sensitivities through the replay", "rsens"
        metric = "replay forward-mode sensitivity trajectories/s (dy1/dtheta on a record) at 1 GPU"
    elif args.mode == "grad_at":
        # the gradient of every accepted step, plus per requested time the
        # reverse of its shortened step (stages and sweep: a gradient step
        # without its forward replay); the sort of the record is part of the call
        fl = steps_total * cfg["grad"] + w.n * STATES_M * (cfg["grad"] - cfg["replay"])
        kern, label, tag = "grad_kernel", f"gradient with cotangents at {STATES_M} times", "gat"
        metric = (f"gradient trajectories/s for a loss on the states at {STATES_M} requested "
                  "times and t1, on a record, 1 GPU")
    else:
        # every lane takes count + m steps of the method (recorded or shortened),
        # each a replay step plus its time update
        fl = (steps_total + w.n * STATES_M) * (cfg["replay"] + 1)
        kern, label, tag = "states_kernel", f"states at {STATES_M} requested times", "states"
        metric = f"trajectories/s for the states at {STATES_M} requested times on a record, 1 GPU"
    ach = fl / tk
    from differentiable_adaptive_ode_amd.profiling import load_traffic

    tr = load_traffic(f"{w.name}_{tag}", w.n)
    traffic = tr["kernels"][kern]["hbm_bytes"] if tr and kern in tr["kernels"] else None
    out = {
        "metric": metric,
        "value": w.n / (wall / args.steps),
        "unit": "trajectories/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} ensemble, {label}", "n_trajectories": w.n,
                   "method": w.method, "t_span": [w.t0, w.t1], "rtol": w.rtol, "atol": w.atol,
                   "s_cap": s_cap, "directions": p if args.mode == "replay_sens" else None,
                   "requested_times": STATES_M if args.mode in ("states", "grad_at") else None},
        "call_ms": tk * 1e3, "accepted_steps_mean": float(cnt.mean()),
        "roofline": {"bound": cfg["bound"], "kernel": kern, "launch_ms": tk * 1e3,
                     "achieved": ach * 1e-12, "peak": cfg["peak"] * 1e-12, "unit": "TFLOP/s",
                     "frac": ach / cfg["peak"], "traffic": traffic,
                     "traffic_unit": "HBM bytes per call"},
        "issue": _issued(tr, kern, fl, w.dtype == "f64"),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_on_record(
            w, args.cpu_sample or min(cfg["cpu_n"], 4096), s_cap, args.mode)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
