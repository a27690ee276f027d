"""Throughput of the fused lattice Boltzmann step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A "step" is one pass of the whole fused step (the in-place AA kernel for
D3Q19 (+D3Q7), bounce-back at walls and solids included; the wall-force pass
on the last step of the submission) over the resident population buffer.
The solver is created first (host link lists, device buffer, the library's
replay graph: the "pipeline creation", timed on its own and reported as
setup_ms), then W untimed steps, then timed regions of exactly K steps in one
submission each, bracketed by stream synchronisation; HIP events on the
library's stream (torch's current stream) time each region.  The line's value
is the mean over the regions (three by default, as the pages quote means of
three runs), with every region and the minimum beside it.

Prints one JSON line: MLUPS (cells * steps / s / 1e6, every cell counted),
the roofline of the dominant kernel (algorithmic HBM bytes per launch / its
average duration over the timed regions, against the 8 TB/s HBM peak; the
kernel's own duration from per-kernel timing after the timed regions beside
it) and the oracle's throughput on the host cores on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLUPS and achieved HBM TB/s, D3Q19(+D3Q7) fp32 AA step, 128³–512³, 1 GPU"
HBM_PEAK_GBPS = 8000.0

# algorithmic bytes per cell update: every population read once and written once
def bytes_per_cell(thermal: bool, dtype: int, streaming: int, two_d: bool = False) -> int:
    q = (9 + (5 if thermal else 0)) if two_d else (19 + (7 if thermal else 0))
    passes = 2 if streaming == 2 else 1  # two buffers in two passes: collide in place, then pull
    return 2 * q * dtype * passes


def hbm_gbps(mlups: float, bytes_per_update: float) -> float:
    """Algorithmic HBM GB/s of a throughput in MLUPS."""
    return mlups * 1e6 * bytes_per_update / 1e9


def mlups_at(gbps: float, bytes_per_update: float) -> float:
    """MLUPS that a bandwidth of gbps GB/s allows at bytes_per_update."""
    return gbps * 1e9 / bytes_per_update / 1e6


WORKLOAD_INFO = {
    "sol256": "D3Q19 MRT isothermal, 256^3 periodic, tau=0.55, seeded random solenoidal velocity "
              "(|u|<=0.05) on rho=1 (the 128^3 in-place/two-buffer recipe at 256^3)",
    "sol128": "D3Q19 MRT isothermal, 128^3 periodic, tau=0.55, seeded random solenoidal velocity (|u|<=0.05)",
    "sol512": "D3Q19 MRT isothermal, 512^3 periodic, tau=0.55, seeded random solenoidal velocity (|u|<=0.05) on "
              "rho=1 (the 128^3 recipe at 512^3)",
    "sphere128": "D3Q19 MRT, 128^3 periodic, centred solid sphere R=16, bounce-back links, gx=1e-6",
    "cavity256": "thermal D3Q19+D3Q7 MRT, 256^3 cavity, x- hot/x+ cold, adiabatic others, Ra=1e7, Pr=0.71",
    "cavity385": "thermal D3Q19+D3Q7 MRT, 385^3 cavity (the thermal-LBM page's 3D grid; it runs fp64), x- hot/x+ "
                 "cold, adiabatic others, Ra=1e7, Pr=0.71",
    "rb512": "thermal D3Q19+D3Q7 MRT, 512^3, periodic x/y, z- hot/z+ cold, random spheres R 4..12 (10%), "
             "Ra=1e8, Pr=0.71",
    "tg32": "D3Q19 MRT, 32^3 periodic Taylor-Green, tau=0.6",
    "channel256": "D3Q19 MRT, 256x128x128 open channel: x- velocity inlet U=0.05, x+ pressure outlet rho=1, "
                  "free-slip y/z faces, solid sphere R=16 at (64,64,64), tau=0.52",
    "cavity2d": "thermal D2Q9+D2Q5 MRT, 8193x8193 square cell, x- hot/x+ cold, adiabatic y faces, no-slip, "
                "Ra=1e8, Pr=0.71, buoyancy +y (the thermal-LBM page's 2D case; it runs fp64)",
    "tg2d": "D2Q9 MRT, 256x256 periodic Taylor-Green, tau=0.6",
}


# streaming mode: (record tag, kernels of one step, description)
STREAMING = {1: ("aa", "k_aa_step", "AA in place"),
             2: ("ab", "k_ab_collide+k_ab_pull", "A-B two buffers, collide then pull"),
             3: ("abpush", "k_ab_push", "A-B two buffers, one pass (collide and push)")}


def kernel_source_hash() -> str:
    """Hash of the library's sources with comments and whitespace removed, so
    that a record of HBM counters stays valid across comment-only edits."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lattice_boltzmann_cfd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, dtype: int, streaming: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else null)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{'f32' if dtype == 4 else 'f64'}"
                        f"_{STREAMING[streaming][0]}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def device_ceilings(nbytes: int = 19 * (1 << 24) * 4, reps: int = 10):
    """Bandwidth of torch's vectorized elementwise kernel out of place (read
    A, write B) and in place (read and write A) on buffers the size of the
    256^3 D3Q19 fp32 population array: the practical ceilings of a copy-like
    and of an in-place access pattern on this GPU."""
    import torch

    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = {}
    for name, fn in (("copy", lambda: torch.mul(a, 1.0, out=b)), ("inplace_rmw", lambda: a.mul_(1.0))):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        out[name + "_GBps"] = round(2 * nbytes * reps / (s.elapsed_time(e) / 1e3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def oracle_stepping_seconds(w, steps: int, threads: int):
    """Wall seconds of `steps` oracle steps on `threads` host threads, less a
    0-step run of the same box (the oracle's serial set-up and read-out)."""
    import oracle

    T = w.T if w.params.get("thermal") else None
    t0 = time.perf_counter()
    oracle.run(w.params, 0, w.rho, w.u, T, labels=w.labels, nthreads=threads)
    t_setup = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.run(w.params, steps, w.rho, w.u, T, labels=w.labels, nthreads=threads)
    dt = time.perf_counter() - t0
    return max(dt - t_setup, 1e-9), dt, t_setup


def cpu_baseline(w, steps: int, steps_one_thread: int):
    """The oracle as it stands on the host cores: `steps` steps on all of
    them and, if asked, `steps_one_thread` steps on one thread."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    oracle.build(force=False)
    stepping, dt, t_setup = oracle_stepping_seconds(w, steps, threads)
    out = {"value": w.cells * steps / stepping / 1e6, "unit": "MLUPS", "cores": threads, "kind": "oracle",
           "sample": f"{steps} steps of the full {w.shape[0]}x{w.shape[1]}x{w.shape[2]} box "
                     f"(fp64 two-buffer collide-then-pull, OpenMP over cells): {dt:.1f} s, less {t_setup:.1f} s "
                     f"of set-up and read-out timed by a 0-step run"}
    if steps_one_thread > 0:
        stepping1, dt1, t_setup1 = oracle_stepping_seconds(w, steps_one_thread, 1)
        out["one_thread"] = {"value": w.cells * steps_one_thread / stepping1 / 1e6, "unit": "MLUPS", "cores": 1,
                             "sample": f"{steps_one_thread} step(s) of the same box on one thread: {dt1:.1f} s, "
                                       f"less {t_setup1:.1f} s of set-up and read-out"}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="sol256", choices=sorted(WORKLOAD_INFO))
    ap.add_argument("--dtype", type=int, default=4, choices=(4, 8))
    ap.add_argument("--streaming", type=int, default=1, choices=(1, 2, 3),
                    help="1 in place (AA), 2 two buffers in two passes, 3 two buffers in one pass")
    ap.add_argument("--cpu-steps", type=int, default=-1,
                    help="oracle steps for the CPU baseline (0: skip; default: 16 at 256^3, about 15 s on 16 host "
                         "threads, as many fewer as the box has more cells, an eighth of that in 2D, at least 1)")
    ap.add_argument("--cpu-steps-one-thread", type=int, default=1,
                    help="oracle steps on one host thread for the same baseline, about 14 s per step at 256^3 "
                         "(0: skip)")
    ap.add_argument("--repeats", type=int, default=3,
                    help="timed regions of K steps: the line's value is their mean; every region and the minimum "
                         "are reported as repeat_MLUPS (the pages quote means of three runs)")
    ap.add_argument("--profile-steps", type=int, default=32,
                    help="after the timed regions, this many more steps with per-kernel timing (lbm_profile): the "
                         "mean milliseconds per launch of each kernel kind, and the step kernel's own roofline "
                         "fraction beside the timed one (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run torch's device copy of 1 GiB 10 times (reference kernel for HBM counters)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU slab decomposition is a design, not code", file=sys.stderr)
        return 2

    import torch

    if args.calibrate_copy:
        # a plain copy of known size: 1 GiB read and 1 GiB written per dispatch
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                          "dispatches": 10}), flush=True)
        return 0

    from lattice_boltzmann_cfd_amd import binding, inputs

    w = inputs.make(args.workload)
    thermal = bool(w.params.get("thermal"))
    # pipeline creation, timed apart from the steps: links on the host, the
    # device buffer, the upload and the library's replay graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    solver = binding.Solver(w.params, w.labels, dtype=args.dtype, streaming=args.streaming)
    torch.cuda.synchronize()
    t_create = time.perf_counter() - t0
    t0 = time.perf_counter()
    solver.init(w.rho, w.u, w.T if thermal else None)
    torch.cuda.synchronize()
    t_init = time.perf_counter() - t0
    stream = torch.cuda.current_stream()
    # the practical ceilings (a device copy and an in-place update of the
    # 256^3 population array's size), measured right before the warm-up: the
    # GPU leaves the idle clocks of the host-side set-up above within ~10 ms
    # of steady load, and a warm-up of a few steps is shorter than that
    practical = device_ceilings()
    solver.step(args.warmup)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    region_ms = []
    for r in range(max(args.repeats, 1)):
        torch.cuda.synchronize()
        start.record(stream)
        solver.step(args.steps)
        end.record(stream)
        torch.cuda.synchronize()
        region_ms.append(start.elapsed_time(end))
        if r == 0:
            # unstable runs raise here (LBM_E_UNSTABLE) rather than report a number
            rho, _, _ = solver.macros()
            solver.wall_force(0)
    runs = [w.cells * args.steps / (ms / 1e3) / 1e6 for ms in region_ms]
    ms = sum(region_ms) / len(region_ms)
    ms_per_step = ms / args.steps
    mlups = sum(runs) / len(runs)

    two_d = int(w.params.get("lattice", 0)) == 1
    bpc = bytes_per_cell(thermal, args.dtype, args.streaming, two_d)
    flow, temp = (9, 5) if two_d else (19, 7)
    has_links = (solver.num_links(flow) + solver.num_links(temp)) > 0
    launches = 2 if args.streaming == 2 else 1
    per_launch_bytes = bpc * w.cells / launches
    # the timed regions hold `launches` bulk kernels per step; the force pass
    # of each submission's last step (and the link passes of a link-pass box)
    # are counted in the step's time as well
    kernel_ms = ms_per_step / launches
    achieved = per_launch_bytes / (kernel_ms / 1e3) / 1e9
    traffic = load_traffic(args.workload, args.dtype, args.streaming)
    kernel = STREAMING[args.streaming][1]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
                "bytes_per_cell": bpc, "bytes_per_launch": int(per_launch_bytes),
                "timing": "HIP events around the timed regions on the library's stream, per launch of the step "
                          "kernel (the gaps between launches included)",
                "launch_includes_links": has_links}

    line = {
        "metric": METRIC, "value": round(mlups, 1), "unit": "MLUPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if args.dtype == 4 else "f64", "data": "synthetic",
        "config": {"workload": args.workload, "description": WORKLOAD_INFO[args.workload],
                   "shape": list(w.shape), "cells": w.cells,
                   "streaming": STREAMING[args.streaming][2],
                   "hbm_TBps_algorithmic": round(hbm_gbps(mlups, bpc) / 1e3, 3)},
        "roofline": roofline,
        "repeat_MLUPS": {"runs": [round(v, 1) for v in runs], "mean": round(mlups, 1), "min": round(min(runs), 1)},
        "setup_ms": {"create": round(t_create * 1e3, 1), "init": round(t_init * 1e3, 1),
                     "note": "solver creation (host link lists and checks, device buffer, upload, the replay graph "
                             "captured and instantiated) and equilibrium initialisation, before any timed step"},
    }
    if args.profile_steps > 0:
        # per-kernel breakdown, outside the timed regions (each kernel launched on its own between events)
        solver.profile(True)
        solver.step(args.profile_steps)
        times = solver.kernel_times()
        solver.profile(False)
        line["kernel_ms"] = {k: round(t / n, 5) for k, (t, n) in times.items()}
        step_kinds = ("ab_collide", "ab_pull") if args.streaming == 2 else ("step_even", "step_odd")
        t_step = sum(times[k][0] for k in step_kinds if k in times)
        n_step = sum(times[k][1] for k in step_kinds if k in times)
        if n_step:
            k_ms = t_step / n_step
            k_gbps = per_launch_bytes / (k_ms / 1e3) / 1e9
            roofline["kernel_profile"] = {"ms_per_launch": round(k_ms, 5), "achieved": round(k_gbps, 1),
                                          "frac": round(k_gbps / HBM_PEAK_GBPS, 4), "launches": n_step}
    if w.labels is not None:
        # solid cells are updated too (on NaN); the throughput over fluid cells only
        fluid = int((w.labels == 0).sum())
        line["config"]["fluid_cells"] = fluid
        line["config"]["fluid_MLUPS"] = round(fluid * args.steps / (ms / 1e3) / 1e6, 1)
    solver.close()
    del rho, solver
    torch.cuda.empty_cache()
    roofline["practical"] = practical
    # about 2.7e8 cell updates in 3D (16 steps at 256^3); the oracle's streaming runs on one thread on a
    # 2D box (one z plane), so an eighth of that there
    budget = 16 * 256 ** 3 // (8 if int(w.params.get("lattice", 0)) == 1 else 1)
    cpu_steps = args.cpu_steps if args.cpu_steps >= 0 else max(1, round(budget / w.cells))
    if cpu_steps > 0:
        line["cpu_baseline"] = cpu_baseline(w, cpu_steps, args.cpu_steps_one_thread)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
