"""Profile bookkeeping for the benchmark: kernel-source digests and summaries of
rocprofv3 CSV output.

    python -m differentiable_adaptive_ode_amd.profiling summarize \\
        --workload lorenz63 --n 65536 --trace DIR --fetch DIR --write DIR \\
        [--sq DIR] --copy-mib 256 --cmd-trace "..." --cmd-fetch "..." \\
        --cmd-write "..." [--cmd-sq "..."] --out profiles

`summarize` reads the kernel_stats / counter_collection CSVs that
`rocprofv3 -f csv` wrote, and writes

* profiles/<workload>_n<N>_kernels.md  -- per-kernel average durations, HBM
  bytes per call and (with --sq) instruction counts, with the commands;
* profiles/traffic_<workload>.json     -- HBM bytes per call of the solve and
  gradient kernels, tagged with the digest of the kernel sources they were
  measured on.

HBM bytes: rocprofv3's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled
by what the same counters read for a plain device-to-device copy of a known
size in the same run (bench.py --copy-calibration MiB): factor = copied bytes /
counted bytes, separately for reads and writes.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def _code_only(text: str) -> str:
    """The source without its comments, whitespace runs collapsed: what the
    compiler sees, so that an edited comment does not invalidate a profile."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # string or character literal, copied whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """sha256 over the HIP sources' code (file names and contents without
    comments, sorted)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def traffic_path(workload: str, root: str | None = None) -> str:
    root = root or os.path.join(os.path.dirname(HERE), "profiles")
    return os.path.join(root, f"traffic_{workload}.json")


def load_traffic(workload: str, n: int):
    """Measured HBM bytes per call for the current kernel sources at ensemble
    size n, or None (no profile, other sources, or another size)."""
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256") != kernel_source_digest() or d.get("n") != n:
        return None
    return d


def _short(name: str) -> str:
    if "solve_kernel" in name and "mlp" not in name:
        # solve_kernel<R, Sys, method, SENS, PHASED>: the variant that integrates
        # the forward sensitivities, the two-phase variant (two launches per
        # solve), or the plain solve
        m = re.search(r", (true|false), (true|false)>\(", name)
        sens = bool(m) and m.group(1) == "true"
        phased = bool(m) and m.group(2) == "true"
        return "solve" + ("_sens" if sens else "") + ("_phased" if phased else "") + "_kernel"
    if "solve_kernel" in name:
        return "solve_kernel"
    if "grad_kernel" in name:
        return "grad_kernel"
    if "states_kernel" in name:
        return "states_kernel"
    if "sens_kernel" in name:
        return "sens_kernel"
    if "mlp" in name.lower():
        return name.split("(")[0].replace("void ", "")
    return name.split("(")[0].replace("void ", "")


def _find(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def read_stats(trace_dir: str):
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_stats.csv"))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["Percentage"])) for r in rows]


def read_counters(d: str):
    """{(kernel name, counter): [values per dispatch]} and {name: grid sizes}."""
    vals = defaultdict(list)
    grids = defaultdict(set)
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        vals[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
        grids[r["Kernel_Name"]].add(int(r["Grid_Size"]))
    return vals, grids


def _copy_counter(vals, counter: str, copy_bytes: int) -> float:
    """Largest per-dispatch value of `counter` over copy kernels (the calibration copy)."""
    best = 0.0
    for (name, c), v in vals.items():
        if c == counter and "copyBuffer" in name:
            best = max(best, max(v))
    if best <= 0:
        raise RuntimeError(f"no copy kernel with {counter} in the counter run")
    return copy_bytes / (best * 1024.0)


def summarize(args) -> None:
    stats = read_stats(args.trace)
    fetch, _ = read_counters(args.fetch)
    write, _ = read_counters(args.write)
    copy_bytes = args.copy_mib << 20
    f_fac = _copy_counter(fetch, "FETCH_SIZE", copy_bytes)
    w_fac = _copy_counter(write, "WRITE_SIZE", copy_bytes)

    def per_launch(vals, counter, fac, key):
        # per call of the library: a two-phase solve is two launches
        xs = [v for (name, c), vv in vals.items() if c == counter and _short(name) == key for v in vv]
        per = 2.0 if "phased" in key else 1.0
        return per * (sum(xs) / len(xs)) * 1024.0 * fac if xs else None

    traffic = {"workload": args.workload, "n": args.n, "kernel_source_sha256": kernel_source_digest(),
               "fetch_factor": f_fac, "write_factor": w_fac, "kernels": {}}
    # (the *_phased_ kernels: the two launches of one two-phase solve together)
    for key in ("solve_kernel", "solve_phased_kernel", "solve_sens_kernel",
                "solve_sens_phased_kernel", "grad_kernel", "sens_kernel", "states_kernel"):
        fb = per_launch(fetch, "FETCH_SIZE", f_fac, key)
        wb = per_launch(write, "WRITE_SIZE", w_fac, key)
        if fb is not None and wb is not None:
            traffic["kernels"][key] = {"read_bytes": fb, "write_bytes": wb, "hbm_bytes": fb + wb}
    os.makedirs(args.out, exist_ok=True)
    with open(traffic_path(args.workload, args.out), "w") as f:
        json.dump(traffic, f, indent=1)

    # Issued floating-point work per call (instruction counters): FP64 lane-flops
    # as 64 x (add + mul + 2 fma + transcendental) wave-instructions, the
    # counter's own FP64 and FP32 flop counts, and MFMA FP32 flops (ops / 512).
    # Against the algorithmic flops of the same call this is the vector units'
    # utilisation under divergence: masked-off lanes and zero-size padding
    # steps are issued but are not work of the method.
    fl = None
    if getattr(args, "flops", None):
        fl, _ = read_counters(args.flops)
        for key, t in traffic["kernels"].items():
            def cnt(c):
                xs = [v for (name, cc), vv in fl.items() if cc == c and _short(name) == key for v in vv]
                per = 2.0 if "phased" in key else 1.0
                return per * sum(xs) / len(xs) if xs else None
            add, mul, fma, trans = (cnt("SQ_INSTS_VALU_ADD_F64"), cnt("SQ_INSTS_VALU_MUL_F64"),
                                    cnt("SQ_INSTS_VALU_FMA_F64"), cnt("SQ_INSTS_VALU_TRANS_F64"))
            if None in (add, mul, fma, trans):
                continue
            mops = cnt("SQ_INSTS_VALU_MFMA_MOPS_F32") or 0.0
            t["issued"] = {"fp64_lane_flops": 64.0 * (add + mul + 2.0 * fma + trans),
                           "fp64_add": add, "fp64_mul": mul, "fp64_fma": fma, "fp64_trans": trans,
                           "counter_flops_fp64": cnt("SQ_INSTS_VALU_FLOPS_FP64"),
                           "counter_flops_fp32": cnt("SQ_INSTS_VALU_FLOPS_FP32"),
                           "mfma_f32_flops": 512.0 * mops}
        with open(traffic_path(args.workload, args.out), "w") as f:
            json.dump(traffic, f, indent=1)

    sq = None
    if args.sq:
        sq, _ = read_counters(args.sq)
    lines = [f"# {args.workload}, n = {args.n}: kernel durations and HBM traffic", "",
             "Kernel trace (rocprofv3 --kernel-trace --stats):", "", "    " + args.cmd_trace, "",
             "| kernel | calls | average us | share of GPU time |", "|---|---|---|---|"]
    for name, calls, avg, pct in stats:
        lines.append(f"| {_short(name)} | {calls} | {avg / 1e3:.2f} | {pct:.1f} % |")
    lines += ["", "HBM bytes per call (FETCH_SIZE, WRITE_SIZE in KiB per dispatch, scaled by the "
              "calibration copy of the same run; a two-phase solve's call is its two launches):",
              "", "    " + args.cmd_fetch, "    " + args.cmd_write, "",
              f"Calibration: a device-to-device copy of {args.copy_mib} MiB reads "
              f"{copy_bytes / f_fac / 1024:.0f} KiB of FETCH_SIZE and {copy_bytes / w_fac / 1024:.0f} KiB of "
              f"WRITE_SIZE, so read bytes = {f_fac:.3f} x FETCH_SIZE x 1024 and write bytes = "
              f"{w_fac:.3f} x WRITE_SIZE x 1024.", "",
              "| kernel | read MB / call | write MB / call |", "|---|---|---|"]
    for key, t in traffic["kernels"].items():
        lines.append(f"| {key} | {t['read_bytes'] / 1e6:.1f} | {t['write_bytes'] / 1e6:.1f} |")
    if sq:
        lines += ["", "Instruction counters (per launch, summed over the device):", "",
                  "    " + args.cmd_sq, ""]
        counters = sorted({c for (_, c) in sq})
        lines.append("| kernel | " + " | ".join(counters) + " |")
        lines.append("|---|" + "---|" * len(counters))
        for key in traffic["kernels"]:
            row = []
            for c in counters:
                xs = [v for (name, cc), vv in sq.items() if cc == c and _short(name) == key for v in vv]
                row.append(f"{sum(xs) / len(xs):.4g}" if xs else "-")
            lines.append(f"| {key} | " + " | ".join(row) + " |")
    if fl:
        lines += ["", "Issued floating-point work per call (instruction counters; FP64 lane-flops = "
                  "64 x (add + mul + 2 fma + transcendental) wave-instructions):", "",
                  "    " + args.cmd_flops, "",
                  "| kernel | FP64 add | FP64 mul | FP64 fma | FP64 trans | FP64 lane-flops | "
                  "SQ_INSTS_VALU_FLOPS_FP64 | SQ_INSTS_VALU_FLOPS_FP32 | MFMA FP32 flops |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for key, t in traffic["kernels"].items():
            iss = t.get("issued")
            if not iss:
                continue
            g = lambda v: "-" if v is None else f"{v:.4g}"  # noqa: E731
            lines.append(f"| {key} | {g(iss['fp64_add'])} | {g(iss['fp64_mul'])} | "
                         f"{g(iss['fp64_fma'])} | {g(iss['fp64_trans'])} | "
                         f"{g(iss['fp64_lane_flops'])} | {g(iss['counter_flops_fp64'])} | "
                         f"{g(iss['counter_flops_fp32'])} | {g(iss['mfma_f32_flops'])} |")
    if getattr(args, "stall", None):
        # Where the wavefronts' cycles go: issuing vector instructions, issuing
        # any instruction, waiting on anything (memory, dependencies), waiting
        # for an instruction to be issued -- each over the wavefronts' lifetime.
        st, _ = read_counters(args.stall)
        lines += ["", "Stall counters (fractions of SQ_WAVE_CYCLES, summed over the device; "
                  "SQ_WAVES wavefronts of the launch):", "", "    " + args.cmd_stall, "",
                  "| kernel | SQ_WAVES | VALU active | any instruction active | waiting (any) | "
                  "waiting for issue | VALU thread utilisation |", "|---|---|---|---|---|---|---|"]
        for key in traffic["kernels"]:
            def c(name):
                xs = [v for (nm, cc), vv in st.items() if cc == name and _short(nm) == key for v in vv]
                return sum(xs) / len(xs) if xs else None
            wc = c("SQ_WAVE_CYCLES")
            if not wc:
                continue
            r = lambda v: "-" if v is None else f"{v / wc:.3f}"  # noqa: E731
            tv, iv = c("SQ_THREAD_CYCLES_VALU"), c("SQ_ACTIVE_INST_VALU")
            util = "-" if not (tv and iv) else f"{tv / (64.0 * iv):.3f}"
            lines.append(f"| {key} | {c('SQ_WAVES'):.0f} | {r(iv)} | {r(c('SQ_ACTIVE_INST_ANY'))} | "
                         f"{r(c('SQ_WAIT_ANY'))} | {r(c('SQ_WAIT_INST_ANY'))} | {util} |")
    lines += ["", f"Kernel sources sha256: `{traffic['kernel_source_sha256']}`", ""]
    path = os.path.join(args.out, f"{args.workload}_n{args.n}_kernels.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(path)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True)
    s.add_argument("--n", type=int, required=True)
    s.add_argument("--trace", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--sq", default=None)
    s.add_argument("--copy-mib", type=int, default=256)
    s.add_argument("--cmd-trace", default="")
    s.add_argument("--cmd-fetch", default="")
    s.add_argument("--cmd-write", default="")
    s.add_argument("--cmd-sq", default="")
    s.add_argument("--flops", default=None)
    s.add_argument("--cmd-flops", default="")
    s.add_argument("--stall", default=None)
    s.add_argument("--cmd-stall", default="")
    s.add_argument("--out", default=os.path.join(os.path.dirname(HERE), "profiles"))
    a = ap.parse_args(argv)
    if a.cmd == "summarize":
        summarize(a)


if __name__ == "__main__":
    main()
