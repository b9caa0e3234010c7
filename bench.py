"""Benchmark: converged state-updates/s of one parallel-in-time solve on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--mode qn]

A step is one complete solve (all iterations, all windows) of a seeded
synthetic workload with inputs resident in HBM.  Default workload: the
channel-wise tanh recurrence s_t = tanh(a*s_{t-1} + x_t), B=8, T=65536, D=256,
float32, quasi-Newton (diagonal Jacobian) to residual 1e-5.

Prints one JSON line.  Besides the throughput it reports the roofline of the
dominant kernel (the steady-state launches of the fused apply kernel, i >= 1,
including the final launch that exits at once; algorithmic bytes = x and s^(i)
read, s^(i+1) written, averaged per launch, over the HIP-event-timed average
launch duration) and the CPU
oracle timed on a bounded sample of the same workload on this host.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "converged state-updates/s (B*T*D) per Newton solve; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
F16_TOL = 1e-3            # residual tolerance with binary16 state storage
FP32_PEAK_TFLOPS = 157.3
MODES = {"jacobi": 0, "picard": 1, "qn": 2, "quasi_newton": 2, "newton": 3, "banded": 4}
KERNEL_SOURCES = {  # source file of the dominant kernel per cell kind
    0: "newton_evaluation_nonlinear_amd/csrc/pn_diag.hip",
    1: "newton_evaluation_nonlinear_amd/csrc/pn_cell.hip",
    2: "newton_evaluation_nonlinear_amd/csrc/pn_cell.hip",
    3: "newton_evaluation_nonlinear_amd/csrc/pn_cell.hip",
}


def _kernel_source(wl, mode):
    dense = mode == 3 or (mode == 4 and 0 < wl["bandwidth"] < wl["D"] - 1)
    # the dense modes run on the matrix cores for D padded to 16 or 32, and to
    # 64 for the single-gate cells (tanh RNN, Euler step)
    mfma = 8 < wl["D"] <= 32 or (32 < wl["D"] <= 64 and wl["cell"] in (1, 3))
    if wl["cell"] != 0 and dense and mfma:
        return "newton_evaluation_nonlinear_amd/csrc/pn_dense.hip"
    return KERNEL_SOURCES[wl["cell"]]


def _src_hash(path):
    with open(os.path.join(ROOT, path), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def _traffic(name, src, launch_bytes_alg):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    they were taken on another revision of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256_16") != _src_hash(src):
        return None
    return t.get("bytes_per_launch")


CPU_SECONDS = 10.0    # CPU work of the oracle baseline (one thread)


def _json_float(v):
    """v, or its name ("inf", "nan") where strict JSON has no number for it."""
    import math
    return float(v) if math.isfinite(v) else str(v)


def _cpu_sample(cfg, mode):
    """The bounded sample of a workload the CPU baselines run (B and T)."""
    samples = {3: dict(B=8, T=32768), 2: dict(B=16, T=2048), 4: dict(B=8, T=4096),
               1: dict(B=None, T=None), 5: dict(B=4, T=4096), 6: dict(B=8, T=4096),
               7: dict(B=None, T=None)}
    if cfg == 2 and mode == 1:
        # float64 Picard on this GRU needs ~T updates (it converges only
        # through its causality bound), so the sample is shorter in time
        return dict(B=16, T=256)
    return samples.get(cfg, dict(B=1, T=4096))


def cpu_baseline(cfg, mode, switch_mode=-1, switch_ratio=0.5, storage=None):
    """The float64 oracle on a bounded sample of the workload, one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads

    wl = workloads.make(cfg, **_cpu_sample(cfg, mode))
    if storage == "f16":
        wl["tol"] = F16_TOL
        wl["x"] = wl["x"].astype(np.float16).astype(np.float32)
    def once():
        if wl["window_mode"] == "advancing":
            cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
            return oracle.solve_advancing(cell, wl["x"], wl["s0"], mode, wl["tol"], wl["max_iter"],
                                          wl["window"], wl["damping"], wl["bandwidth"])
        return oracle.solve(wl["cell"], wl["params"], wl["x"], wl["s0"], mode, wl["tol"],
                            wl["max_iter"], wl["damping"], wl["window"], bandwidth=wl["bandwidth"],
                            switch_mode=switch_mode if switch_mode >= 0 else None,
                            switch_ratio=switch_ratio, storage=storage)

    # the sample solve, repeated until it has taken CPU_SECONDS on one thread
    reps, el = 0, 0.0
    with threadpool_limits(1):
        while el < CPU_SECONDS and reps < 20000:
            t0 = time.perf_counter()
            r = once()
            el += time.perf_counter() - t0
            reps += 1
    n = wl["B"] * wl["T"] * wl["D"]
    return {"value": reps * n / el, "unit": "state-updates/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 oracle solve of the same workload cut to B={wl['B']}, "
                      f"T={wl['T']} (D={wl['D']}): {r.iters} updates, status {r.status}; "
                      f"{reps} runs, {el:.1f} s on one host thread",
            "seconds": el}


# ---------------------------------------------------------------- CPU detail
# Inherited by forked workers (no pickling of the sample arrays).
_DETAIL = {}


def _detail_rows(job):
    """One worker of the batch split: the rows [b0, b1) of the sample."""
    from threadpoolctl import threadpool_limits
    import oracle
    what, b0, b1 = job
    d = _DETAIL
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if what == "sequential":
            oracle.sequential(d["cell"], d["x64"][b0:b1], d["s064"][b0:b1])
        elif d["wl"]["window_mode"] == "advancing":
            wl = d["wl"]
            oracle.solve_advancing(d["cell"], wl["x"][b0:b1], wl["s0"][b0:b1], d["mode"], wl["tol"],
                                   wl["max_iter"], wl["window"], wl["damping"], wl["bandwidth"])
        else:
            wl = d["wl"]
            oracle.solve(wl["cell"], wl["params"], wl["x"][b0:b1], wl["s0"][b0:b1], d["mode"], wl["tol"],
                         wl["max_iter"], wl["damping"], wl["window"], bandwidth=wl["bandwidth"],
                         switch_mode=d["switch_mode"], switch_ratio=d["switch_ratio"],
                         storage=d["storage"])
        return time.perf_counter() - t0


def cpu_detail(cfg, mode, switch_mode=-1, switch_ratio=0.5, storage=None):
    """The float64 sequential loop and the float64 oracle solve on the CPU
    baseline's sample: each on one core, then split across the batch rows
    over the host's cores (forked workers, one row range each).  The split
    solves stop on their own rows' residuals, not the batch-global rule."""
    import multiprocessing as mp
    import numpy as np
    import oracle
    import workloads

    wl = workloads.make(cfg, **_cpu_sample(cfg, mode))
    if storage == "f16":
        wl["tol"] = F16_TOL
        wl["x"] = wl["x"].astype(np.float16).astype(np.float32)
    cell = oracle.make_cell(wl["cell"], wl["params"], wl["D"], wl["m"])
    _DETAIL.clear()
    _DETAIL.update(wl=wl, cell=cell, mode=mode, storage=storage, switch_ratio=switch_ratio,
                   switch_mode=switch_mode if switch_mode >= 0 else None,
                   x64=wl["x"].astype(np.float64), s064=wl["s0"].astype(np.float64))
    B = wl["B"]
    n = wl["B"] * wl["T"] * wl["D"]
    cores = len(os.sched_getaffinity(0))
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    out = {"cores_available": cores, "cpu_model": model,
           "sample": f"B={B}, T={wl['T']}, D={wl['D']} of the same workload"}
    single = {}
    for what in ("sequential", "solve"):
        el = _detail_rows((what, 0, B))
        single[what] = {"seconds": el, "state_updates_per_s": n / el}
    out["single_core"] = single
    workers = min(cores, B, 16)
    edges = [B * k // workers for k in range(workers + 1)]
    split = {"workers": workers}
    with mp.get_context("fork").Pool(workers) as pool:
        for what in ("sequential", "solve"):
            t0 = time.perf_counter()
            pool.map(_detail_rows, [(what, edges[k], edges[k + 1]) for k in range(workers)])
            el = time.perf_counter() - t0
            split[what] = {"seconds": el, "state_updates_per_s": n / el}
    out["batch_split"] = split
    _DETAIL.clear()
    return out


CEILING_BYTES = 512 << 20      # per array: the headline's x (8 x 65536 x 256 floats)
CEILING_PATTERNS = (("read", 0), ("write", 1), ("copy", 2), ("2r1w_flat", 3), ("2r1w_rows", 4), ("read_rows", 5))


def ceilings(reps=10):
    """Measured ceilings of this GPU from libpn_ceiling.so (include/pn_ceiling.h):
    GB/s of plain streaming kernels and TFLOP/s of a plain FP32 matrix-core
    loop, best and median of `reps` event-timed launches."""
    import ctypes
    path = os.path.join(ROOT, "newton_evaluation_nonlinear_amd", "libpn_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build with `python -m newton_evaluation_nonlinear_amd._build`")
    L = ctypes.CDLL(path)
    dbl = ctypes.c_double
    L.pnc_hbm.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
    L.pnc_mfma_f32.argtypes = [ctypes.c_int, ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
    L.pnc_last_error.restype = ctypes.c_char_p
    out = {"unit": "GB/s", "bytes_per_array": CEILING_BYTES, "reps": reps}
    for name, pat in CEILING_PATTERNS:
        best, med = dbl(0.0), dbl(0.0)
        if L.pnc_hbm(pat, CEILING_BYTES, reps, ctypes.byref(best), ctypes.byref(med)) != 0:
            raise SystemExit("ceiling microbenchmark failed: " + L.pnc_last_error().decode())
        out[name] = {"best": best.value, "median": med.value}
    best, med = dbl(0.0), dbl(0.0)
    if L.pnc_mfma_f32(reps, ctypes.byref(best), ctypes.byref(med)) != 0:
        raise SystemExit("ceiling microbenchmark failed: " + L.pnc_last_error().decode())
    out["mfma_f32_tflops"] = {"best": best.value, "median": med.value}
    return out


def sequential_gpu(params, x, s0, out_solve, solve_ms, reps=10):
    """The plain time loop of the channel-wise cell on the same GPU and the
    same inputs (libpn_ceiling.so, pnc_sequential_tanh: one thread per (b, d)
    walking t in order): the GPU baseline of the parallel-in-time solve, with
    its largest difference from the solve's trajectory."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "newton_evaluation_nonlinear_amd", "libpn_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build with `python -m newton_evaluation_nonlinear_amd._build`")
    L = ctypes.CDLL(path)
    vp, dbl = ctypes.c_void_p, ctypes.c_double
    L.pnc_sequential_tanh.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
    L.pnc_last_error.restype = ctypes.c_char_p
    B, T, D = out_solve.shape
    seq = torch.empty_like(out_solve)
    torch.cuda.synchronize()
    best, med = dbl(0.0), dbl(0.0)
    if L.pnc_sequential_tanh(x.data_ptr(), params.data_ptr(), s0.data_ptr(), seq.data_ptr(), B, T, D, reps,
                             ctypes.byref(best), ctypes.byref(med)) != 0:
        raise SystemExit("sequential GPU loop failed: " + L.pnc_last_error().decode())
    diff = float((seq - out_solve).abs().max())
    return {"kernel": "time loop in order, one thread per (b, d) (pnc_sequential_tanh)",
            "ms": med.value, "best_ms": best.value,
            "state_updates_per_s": B * T * D / (med.value * 1e-3),
            "solve_ms": solve_ms, "solve_speedup_over_loop": med.value / solve_ms,
            "max_abs_diff_vs_solve": diff}


COPY_PROBE_BYTES = 64 * 1024 * 1024 * 4   # read once and written once by the probe copy


def _read_counters(d, counter):
    """{dispatch_id: (kernel_name, value)} from a rocprofv3 counter_collection csv."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                did = int(row["Dispatch_Id"])
                name, val = out.get(did, (row["Kernel_Name"], 0.0))
                out[did] = (name, val + float(row["Counter_Value"]))
    return out


def _steady_apply(kernel_name):
    """True for a steady-state apply launch (phase template argument 2), from
    the demangled name or, where the profiler leaves it mangled, from the
    integer template arguments (Li<n>E) of the mangled one."""
    import re
    m = re.search(r"\b(diag_tanh_pass|cell_pass|dense_pass)<([^>]*)>", kernel_name)
    if m:
        targs = [a.strip() for a in m.group(2).split(",")]
        pos = {"diag_tanh_pass": 1, "cell_pass": 3, "dense_pass": 2}[m.group(1)]
        return len(targs) > pos and targs[pos] == "2"
    m = re.search(r"\d+(diag_tanh_pass|cell_pass|dense_pass)I(.*)", kernel_name)
    if not m:
        return False
    ints = re.findall(r"Li(\d+)E", m.group(2))
    pos = {"diag_tanh_pass": 1, "cell_pass": 2, "dense_pass": 2}[m.group(1)]
    return len(ints) > pos and ints[pos] == "2"


def summarize_pmc(args, fetch_dir, write_dir):
    """Per-launch HBM bytes of the dominant kernel from two counter runs.

    FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch; both are scaled
    by the ratio of the known bytes of the probe copy to what the same counter
    reads for it."""
    import workloads
    wl = workloads.make(args.config, B=1, T=1)   # names only
    mode = MODES[args.mode] if args.mode else wl["modes"][0]
    name = f"{wl['name']}_{workloads.MODE_NAMES[mode]}" + ("_f16" if args.storage == "f16" else "")
    res = {}
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _read_counters(d, counter)
        copies = [v for n, v in rows.values() if "copyBuffer" in n]   # the device-to-device probe
        if not copies:
            raise SystemExit(f"no copy-probe dispatch found in {d}")
        scale = COPY_PROBE_BYTES / (max(copies) * 1024.0)
        steady = [v for n, v in rows.values() if _steady_apply(n)]
        if not steady:
            raise SystemExit(f"no steady apply dispatch found in {d}")
        per = sum(steady) / len(steady) * 1024.0
        res[label] = dict(counter=counter, copy_probe_kib=max(copies), scale=scale,
                          launches=len(steady), raw_bytes_per_launch=per,
                          bytes_per_launch=per * scale)
    src = _kernel_source(wl, mode)
    bargs = f"--config {args.config}" + (f" --mode {args.mode}" if args.mode else "") + \
        (" --storage f16" if args.storage == "f16" else "")
    cmds = [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- "
            f"python3 bench.py {bargs} --steps 2 --warmup 0 --no-cpu --copy-probe",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- "
            f"python3 bench.py {bargs} --steps 2 --warmup 0 --no-cpu --copy-probe",
            f"python3 bench.py {bargs} --pmc-summary {fetch_dir} {write_dir}"]
    out = dict(workload=name, commands=cmds, kernel="steady apply launches", source=src,
               source_sha256_16=_src_hash(src),
               bytes_per_launch=res["fetch"]["bytes_per_launch"] + res["write"]["bytes_per_launch"],
               fetch=res["fetch"], write=res["write"])
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def scan_bench(reps=20):
    """The exported scan step alone (pn_affine_scan) on the headline's shape
    (diagonal A, B=8, T=65536, D=256) and a dense one (B=4, T=4096, D=64):
    time per call (host-timed, blocking) and the algorithmic rate: A and b read
    once, out written once."""
    import numpy as np
    import torch
    import newton_evaluation_nonlinear_amd as pn
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(5)
    res = {}
    for name, (B, T, D, dense) in (("diag_b8_t65536_d256", (8, 65536, 256, False)),
                                   ("dense_b4_t4096_d64", (4, 4096, 64, True))):
        shape = (B, T, D, D) if dense else (B, T, D)
        A = torch.rand(shape, device=dev, generator=gen) * (0.45 / (D ** 0.5 if dense else 1.0)) + \
            (0.0 if dense else 0.5)
        b = torch.randn((B, T, D), device=dev, generator=gen)
        s0 = torch.randn((B, D), device=dev, generator=gen)
        out = torch.empty_like(b)
        for _ in range(3):
            pn.affine_scan(A, b, s0, dense=dense, out=out)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            pn.affine_scan(A, b, s0, dense=dense, out=out)
            ts.append(time.perf_counter() - t0)
        ts.sort()
        med = ts[len(ts) // 2]
        nbytes = 4.0 * (A.numel() + b.numel() + out.numel())
        res[name] = {"ms_median": med * 1e3, "alg_gbs": nbytes / med / 1e9,
                     "frac_of_8tbs": nbytes / med / 8e12, "alg_bytes": nbytes,
                     "dense": dense, "B": B, "T": T, "D": D}
        del A, b, s0, out
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--mode", default=None)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--switch", default=None,
                    help="residual-driven switching: the mode each window moves to on a stall")
    ap.add_argument("--switch-ratio", type=float, default=0.5)
    ap.add_argument("--storage", choices=("f32", "f16"), default="f32",
                    help="f16: x and the iterate stored in binary16 (channel-wise cell), "
                         "float32 arithmetic, tol 1e-3")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU baselines (cpu_baseline and cpu_detail)")
    ap.add_argument("--cpu-detail", action="store_true", help=argparse.SUPPRESS)   # now the default
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the ceiling microbenchmarks (libpn_ceiling.so)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 256 MiB device copy first (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-probe` into profiles/<workload>_traffic.json")
    ap.add_argument("--scan", action="store_true",
                    help="time the exported scan step alone (pn_affine_scan) and print one JSON line")
    args = ap.parse_args()
    if args.scan:
        print(json.dumps({"scan": scan_bench()}), flush=True)
        return
    if args.pmc_summary:
        summarize_pmc(args, *args.pmc_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described, not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import newton_evaluation_nonlinear_amd as pn

    wl = workloads.make(args.config)
    mode = MODES[args.mode] if args.mode else wl["modes"][0]
    half = args.storage == "f16"
    if half:
        # binary16 states cannot meet 1e-5: their spacing below 1 is 4.9e-4
        wl["tol"] = F16_TOL
        wl["x"] = wl["x"].astype(np.float16)
    dev = torch.device("cuda:0")
    params, x, s0 = (torch.from_numpy(wl[k]).to(dev) for k in ("params", "x", "s0"))
    out = torch.empty((wl["B"], wl["T"], wl["D"]), dtype=torch.float16 if half else torch.float32,
                      device=dev)
    wmode = pn.WINDOW_ADVANCING if wl["window_mode"] == "advancing" else pn.WINDOW_CONSECUTIVE
    smode = MODES[args.switch] if args.switch else -1
    nbytes = pn.workspace_bytes(wl["cell"], wl["m"], wl["B"], wl["T"], wl["D"], mode,
                                wl["damping"], wl["window"], args.chunk, wl["bandwidth"], wmode,
                                smode)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)

    def solve(profile):
        return pn.eval(wl["cell"], params, x, s0, mode=mode, tol=wl["tol"],
                       max_iter=wl["max_iter"], damping=wl["damping"], window=wl["window"],
                       chunk=args.chunk, out=out, workspace=ws, profile=profile, history=True,
                       bandwidth=wl["bandwidth"], window_mode=wmode, switch_mode=smode,
                       switch_ratio=args.switch_ratio)

    if args.copy_probe:
        n = 64 * 1024 * 1024
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # Timing events cost several microseconds per timed launch (about 6.5 us
    # on a 15 us launch), so a solve of many launches times a sample of
    # about four of them (every n-th steady launch); the launches of a solve
    # are alike, and the timed steps give tens of samples.  The last warm-up
    # solve (from the second on) times launches too, so that the events
    # exist before the timed region.
    # A solve of only a few launches (the one-workgroup solver: one) would
    # spend a large share of its wall time on the events, so there only every
    # `every`-th timed step carries them.
    warm, every = None, 1
    for k in range(args.warmup):
        if k == args.warmup - 1 and warm is not None:
            wp = solve(max(1, warm.iters // 4))
            every = 1 if wp.profile["apply_launches"] >= 4 else 8
        else:
            warm = solve(False)
    torch.cuda.synchronize()
    stride = max(1, (warm.iters if warm is not None else 0) // 4)
    results, step_ms = [], []
    t0 = time.perf_counter()
    for k in range(args.steps):
        ts = time.perf_counter()
        results.append(solve(stride if k % every == 0 else False))   # returns once its stream is idle
        step_ms.append((time.perf_counter() - ts) * 1e3)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) / args.steps * 1e3
    n_upd = wl["B"] * wl["T"] * wl["D"]
    value = n_upd / (ms / 1e3)
    last = results[-1]
    prof = [r.profile for r in results if r.profile is not None]
    apply_ms = sum(p["apply_ms"] for p in prof)
    apply_launches = sum(p["apply_launches"] for p in prof)
    apply_bytes = sum(p["apply_bytes"] for p in prof)
    apply_flops = sum(p["apply_flops"] for p in prof)
    avg_launch_ms = apply_ms / max(apply_launches, 1)
    bytes_per_launch = apply_bytes / max(apply_launches, 1)
    gbs = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9 if avg_launch_ms > 0 else 0.0
    name = f"{wl['name']}_{workloads.MODE_NAMES[mode]}" + ("_f16" if half else "")
    if smode >= 0:
        name += f"_to_{workloads.MODE_NAMES[smode]}"
    src = _kernel_source(wl, smode if smode >= 0 else mode)
    # bound by arithmetic intensity of the kernel against the FP32 ridge point
    flops_per_launch = apply_flops / max(apply_launches, 1)
    if flops_per_launch > bytes_per_launch * (FP32_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9):
        tf = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
        # the dense modes outside the matrix-core kernel compose on the vector
        # ALUs (FP32 vector and matrix peaks are both 157.3 TFLOP/s on MI355X)
        fine = smode if smode >= 0 else mode
        dense = fine == 3 or (fine == 4 and 0 < wl["bandwidth"] < wl["D"] - 1)
        # at D padded to 64 a band of at most two diagonals each side extends
        # the chunk map on the vector ALUs (the row chain of dense64_pass)
        row_chain = (fine == 4 and 0 < wl["bandwidth"] <= 2 and wl["bandwidth"] < wl["D"] - 1 and
                     32 < wl["D"] <= 64 and wl["cell"] in (1, 3))
        unit = "alu" if dense and (src == KERNEL_SOURCES[wl["cell"]] or row_chain) else "mfma"
        roof = {"bound": unit, "achieved": tf, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / FP32_PEAK_TFLOPS, "traffic": _traffic(name, src, bytes_per_launch)}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": _traffic(name, src, bytes_per_launch)}
    roof.update(kernel="apply (fused cell + scan replay + residual + next chunk maps)",
                avg_launch_ms=avg_launch_ms, timed_launches_per_step=apply_launches / max(len(prof), 1),
                timed_every=stride, timed_steps=len(prof),
                alg_bytes_per_launch=bytes_per_launch, alg_flops_per_launch=flops_per_launch)
    line = {
        "metric": METRIC, "value": value, "unit": "state-updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_median": sorted(step_ms)[len(step_ms) // 2],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 arithmetic, f16 storage" if half else "f32",
        "data": "synthetic (seeded PCG64 draws, no dataset)",
        "config": {"workload": name, "cell": wl["cell"], "B": wl["B"], "T": wl["T"],
                   "D": wl["D"], "m": wl["m"], "mode": workloads.MODE_NAMES[mode],
                   "tol": wl["tol"], "damping": wl["damping"], "window": wl["window"],
                   **({"window_mode": "advancing"} if wmode else {}),
                   **({"bandwidth": wl["bandwidth"]} if 4 in (mode, smode) else {}),
                   **({"switch_to": workloads.MODE_NAMES[smode], "switch_ratio": args.switch_ratio,
                       "window_switch_first": last.window_switch[:4]} if smode >= 0 else {}),
                   "iters": last.iters, "window_iters_first": last.window_iters[:4],
                   "final_residual": _json_float(last.resid_hist[-1]) if last.resid_hist else None,
                   "status": last.status, "parallelism": "single GPU"},
        "roofline": roof,
    }
    if not args.no_ceiling:
        ceil = ceilings()
        line["ceilings"] = ceil
        if roof["bound"] == "hbm":
            # the pattern of the steady apply kernel: two row streams in, one out
            c = ceil["2r1w_rows"]["median"]
            roof.update(measured_ceiling={"pattern": "2r1w_rows", "value": c, "unit": "GB/s"},
                        frac_of_measured_ceiling=roof["achieved"] / c)
        elif roof["bound"] == "mfma":
            c = ceil["mfma_f32_tflops"]["median"]
            roof.update(measured_ceiling={"pattern": "mfma_f32", "value": c, "unit": "TFLOP/s"},
                        frac_of_measured_ceiling=roof["achieved"] / c)
    if not args.no_ceiling and wl["cell"] == 0 and not half and not wmode and wl["window"] == 0:
        line["sequential_gpu"] = sequential_gpu(params, x, s0, out, ms)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.config, mode, smode, args.switch_ratio,
                                            "f16" if half else None)
        line["cpu_detail"] = cpu_detail(args.config, mode, smode, args.switch_ratio,
                                        "f16" if half else None)
        line["cpu_detail"]["context"] = ("the article's A100 timings of an unspecified T=2048 RNN "
                                         "forward: sequential 12.3 ms, Picard 4.2 ms, quasi-Newton 3.1 ms")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
