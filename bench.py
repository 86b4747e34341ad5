"""Throughput of the GSQ relaxed-quantization step on one MI355X.

A step is one pass of the whole hot path over the layer: relaxed forward
(soft weights, dW), reconstruction loss and gradient (two bf16 MFMA
products), relaxed backward with the fused Lion update. The headline
workload is the largest one that fits one GPU: a mixture-of-experts batch of
64 experts, each W 2048x7168 bf16 ~N(0, 0.02^2) on the 2-bit grid (four fp32
logits per weight, group-128 scales), each with its own routed calibration
tokens (counts drawn from Zipf(1.1) on [64, 1024], bf16 N(0,1) rows of 7168),
Lion lr 1e-3; the reconstruction products run as one grouped launch each.

Prints one JSON line: weights/s over the timed steps, per-call times from HIP
events recorded on the launch stream, the roofline of the dominant kernel,
the CPU oracle's rate on a bounded sample of the same workload, and the same
step measured on the other synthetic layers (``variants``: the Llama-3.1-8B
q_proj and down_proj shapes and the 70B gate_proj shape).
``--workload`` makes another layer the headline. ``--traffic`` turns two
rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) of this script into the
per-launch HBM bytes under ``profiles/`` (no GPU needed for that step).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
WORKLOAD = "moe64x2048x7168_int2"
VARIANTS = ("qproj4096_int2", "downproj4096x14336_ternary", "gateproj28672x8192_int3local")
N_LOGITS = {0: 4, 1: 2, 2: 5, 3: 8}    # 2-bit, ternary, 3-bit local shift, full 3-bit


def bytes_per_coord(grid: int, w_bf16: bool) -> dict:
    """Bytes per weight coordinate per call. Forward: L fp32 logits + W read,
    dW (bf16) written. Backward + Lion: G, L logits and L momenta read, L
    logits and L momenta written. The fused backward + next forward adds W
    and dW. Local shift also reads its 1-byte warm-start code (once in the
    fused pass). Group scale traffic (< 0.2 B) is left out. 2-bit bf16:
    20 / 68 / 72 B. ``step`` is the relax work of one step as the method
    defines it (forward + backward + Lion, each reading its own inputs:
    fwd + bwd, 88 B at 2-bit bf16), which the fused pass does while moving
    ``fused`` bytes."""
    L = N_LOGITS[grid]
    wb = 2 if w_bf16 else 4
    code = 1 if grid == 2 else 0
    fwd, bwd = 4 * L + wb + 2 + code, 4 + 16 * L + code
    return {"fwd": fwd, "bwd": bwd, "fused": 4 + 16 * L + wb + 2 + code, "step": fwd + bwd}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


# The sources the relax kernels (the dominant kernel's family) are built from.
RELAX_SOURCES = ("gsq_device.hpp", "gsq_internal.hpp", "relax_device.hpp", "relax.hip",
                 "fused.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "post_weight_quantization_philox_amd", "csrc")
    for fn in RELAX_SOURCES:
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def host_info() -> dict:
    """The host the oracle ran on: CPU model, logical CPUs, the affinity mask's
    size and the thread-count environment variables."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                      "MKL_NUM_THREADS") if k in os.environ}
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "affinity": affinity,
            "thread_env": env}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:            # threadpoolctl missing: report one thread
        return 1


def cpu_baseline(data, rows: int = 0, experts: int = 0):
    """The oracle (NumPy fp64) on a bounded sample of the workload: one full
    step (relaxed forward, both products, backward, Lion on logits and
    scales) on the first ``rows`` rows of a dense layer against all its
    tokens, or on the first ``experts`` whole experts of a batch, each
    against its own routed tokens (its rows placed at their rows in the
    batch for the noise counters)."""
    import numpy as np
    import oracle
    blas_threads = _blas_threads()
    wl = data["workload"]
    X = data["X"]
    if wl.experts > 1:
        rpe = wl.rows_per_expert
        offs = data["tok_offsets"]
        n_w, dt, toks = 0, 0.0, 0
        for e in range(experts):
            W = data["W"][e * rpe:(e + 1) * rpe]
            Xe = X[offs[e]:offs[e + 1]]
            scales, codes, logits = oracle.init_rtn(W, wl.grid)
            state = {"logits": logits, "mom": np.zeros_like(logits), "scales": scales,
                     "scale_mom": np.zeros_like(scales), "codes": codes}
            t0 = time.perf_counter()
            oracle.step(state, W, Xe, wl.grid, 0, 1.0, 0, 0, 1e-3, 1e-5, bf16_dW=True,
                        row0=e * rpe)
            dt += time.perf_counter() - t0
            n_w += W.size
            toks += Xe.shape[0]
        sample = (f"one full step on experts 0..{experts - 1} of the {wl.experts}-expert batch "
                  f"({n_w} weights, {toks} routed tokens in all), {dt:.1f} s")
    else:
        W = data["W"][:rows]
        scales, codes, logits = oracle.init_rtn(W, wl.grid)
        state = {"logits": logits, "mom": np.zeros_like(logits), "scales": scales,
                 "scale_mom": np.zeros_like(scales), "codes": codes}
        t0 = time.perf_counter()
        oracle.step(state, W, X, wl.grid, 0, 1.0, 0, 0, 1e-3, 1e-5, bf16_dW=True)
        dt = time.perf_counter() - t0
        n_w = W.size
        sample = (f"one full step on rows 0..{rows - 1} of the {wl.rows}x{wl.cols} layer "
                  f"({n_w} weights) against all {X.shape[0]} tokens, {dt:.1f} s")
    return {"value": n_w / dt, "unit": "weights/s", "cores": blas_threads,
            "kind": "oracle", "host": host_info(),
            "sample": sample + f"; NumPy elementwise work on one thread, BLAS on {blas_threads}"}


def describe(wl) -> str:
    grid = {0: "2-bit grid (4 fp32 logits/weight)", 1: "ternary mask+sign (2 fp32 logits/weight)",
            2: "3-bit local shift (5 fp32 logits/weight)",
            3: "3-bit full grid (8 fp32 logits/weight)"}[wl.grid]
    x = {"normal": "N(0,1)", "normal_outliers": "N(0,1) with 1% outlier channels x20",
         "student_t4": "Student-t(4)"}[wl.x_kind]
    w = "bf16" if wl.w_bf16 else "fp32"
    if wl.experts > 1:
        return (f"{wl.experts} experts of {wl.rows_per_expert}x{wl.cols} {w}, {grid}, group 128, "
                f"routed tokens per expert ~ Zipf({wl.extra['zipf_a']}) on "
                f"[{wl.extra['n_min']}, {wl.extra['n_max']}], bf16 {x}")
    return f"{wl.rows}x{wl.cols} {w}, {grid}, group 128, {wl.tokens} tokens bf16 {x}"


SPIN_UP_S = 0.5


def spin_up(step_fn):
    """Untimed steps for SPIN_UP_S seconds of wall time before the warm-up
    steps: the GPU's clocks take longer than a few milliseconds of work to
    settle, and the timed steps should see the steady state."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SPIN_UP_S:
        for _ in range(10):
            step_fn()
        torch.cuda.synchronize()


def time_fused(solver, taus, warmup: int, steps: int, stream):
    """Fused-step timing loop: returns (elapsed s, mean ms of the first call,
    mean ms of the second). Step t = objective of step t (dW from the
    previous pass) + backward and Lion of step t fused with the forward of
    step t + 1. With the solver's fused product (``solver.fuse``) the calls
    are the first product (R^T) and the second product fused with the
    backward; otherwise both products, then the fused relax pass."""
    import numpy as np
    import torch
    # The spin-up steps change the state; the timed steps start from the
    # warm start again, so every run times the same trajectory.
    start = solver.state()
    solver.relax_fwd(0, taus[0])
    spin_up(lambda: solver.step_fused(0, taus[0], taus[1]))
    solver.load_state(start)
    del start
    solver.relax_fwd(0, taus[0])
    for t in range(warmup):
        solver.step_fused(t, taus[t], taus[t + 1])
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        t = warmup + i
        e = ev[i]
        e[0].record(stream)
        if solver.fuse:
            solver.recon_residual()
            e[1].record(stream)
            solver.recon_bwd_lion_fwd(t, taus[t], taus[t + 1])
        else:
            solver.recon()
            e[1].record(stream)
            solver.relax_bwd_lion_fwd(t, taus[t], t + 1, taus[t + 1])
        e[2].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    first_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    second_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    return elapsed, first_ms, second_ms


def block_bench(args, dev):
    """GSQ's staged schedule (query/key, value/output, MLP) over one decoder
    block of Llama-3.1-8B shape with seeded random weights and 4096 tokens of
    N(0,1) activations: weights/s = all projection weights x steps per layer /
    wall time of the whole schedule (forwards, set-up, solves, hardening)."""
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.block import LLAMA3_8B, staged_quantize
    cfg = LLAMA3_8B
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    w = {}
    for name, (o, i) in cfg.shapes().items():
        w[name] = (torch.randn((o, i), generator=gen, device=dev) / i ** 0.5).to(torch.bfloat16)
    w["g_attn"] = torch.ones(cfg.hidden, device=dev)
    w["g_mlp"] = torch.ones(cfg.hidden, device=dev)
    x = torch.randn((4096, cfg.hidden), generator=gen, device=dev).to(torch.bfloat16)
    lion = g.GsqLion.make(lr_logit=1e-3, lr_scale=1e-5)
    staged_quantize(cfg, w, x[:256], g.GRID_INT2, 2, lion, recon=args.block_recon,
                    objective=args.block_objective)   # warm up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, info = staged_quantize(cfg, w, x, g.GRID_INT2, args.block_steps, lion,
                              recon=args.block_recon, objective=args.block_objective)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    n_w = sum(o * i for o, i in cfg.shapes().values())
    print(json.dumps({
        "metric": "GSQ staged block schedule weights/sec (all projections x steps)",
        "value": n_w * args.block_steps / el, "unit": "weights/s", "n_gpus": 1,
        "steps": args.block_steps, "seconds": el, "higher_is_better": True, "data": "synthetic",
        "dtype": "f32 relax+Lion, bf16 MFMA (fp32 accumulate), bf16 block forward",
        "config": {"workload": "Llama-3.1-8B-shaped decoder block (hidden 4096, 32 heads, 8 kv "
                               "heads, MLP 14336), random weights, 4096 tokens N(0,1), 2-bit grid",
                   "weights": n_w, "recon": args.block_recon,
                   "objective": args.block_objective},
        "stages": {k: {"seconds": v["seconds"], "recon": v["recon"]} for k, v in info.items()},
    }), flush=True)


def _kernel_names():
    """rocprofv3 kernel-name prefixes of the step's calls."""
    return {"relax_bwd_lion_fwd": "relax_bwd_lion_kernel", "relax_fwd": "relax_fwd_kernel",
            "relax_bwd_lion": "relax_bwd_lion_kernel"}


def write_traffic(workload: str, fetch_dir: str, write_dir: str):
    """HBM bytes per launch of every kernel of a workload's bench run, from
    two rocprofv3 counter runs of ``bench.py --workload W`` (``--pmc
    FETCH_SIZE``, then ``--pmc WRITE_SIZE``; both in KiB per dispatch).
    Each counter is scaled by what it reads for the run's calibration copy
    (``neg`` of a 256 MiB fp32 tensor into another: 256 MiB read, 256 MiB
    written). Writes ``profiles/traffic_<workload>.json`` with the hash of
    the relax kernels' sources."""
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        acc = {}
        for fn in files:
            with open(fn) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return acc

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    cal = [k for k in fetch if "neg_kernel" in k]
    if len(cal) != 1:
        raise SystemExit(f"calibration copy not found once among the kernels: {cal}")
    true_kib = 256 * 1024.0
    ff = true_kib / (sum(fetch[cal[0]]) / len(fetch[cal[0]]))
    wf = true_kib / (sum(write[cal[0]]) / len(write[cal[0]]))
    out = {"source_hash": kernel_source_hash(), "fetch_factor": ff, "write_factor": wf,
           "calibration": "neg of a 256 MiB fp32 tensor (256 MiB read, 256 MiB written)",
           "command": (f"rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o pmc -- python3 bench.py "
                       f"--workload {workload} --steps 3 --warmup 1 --no-variants --no-cpu-baseline "
                       f"--no-ab; the same with --pmc WRITE_SIZE -d {write_dir}; then python3 "
                       f"bench.py --workload {workload} --traffic {fetch_dir} {write_dir}"),
           "kernels": {}}
    for k in sorted(set(fetch) & set(write)):
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        out["kernels"][k] = {"dispatches": len(fetch[k]), "fetch_kib_raw": fk, "write_kib_raw": wk,
                             "bytes_per_launch": 1024.0 * (fk * ff + wk * wf)}
    with open(traffic_file(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(traffic_file(workload))


def measured_kernel_traffic(workload: str, call: str):
    """Counter bytes per launch of the kernel behind a bench call (the
    fused pass: the relax_bwd_lion kernel instantiated with the next
    forward), or None if no counter run matches the current sources."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    if call in t.get("kernels", {}):                 # older files: keyed by call
        return t["kernels"][call].get("bytes_per_launch")
    # Template arguments: relax_bwd_lion_kernel<grid, debug, next forward, ...>,
    # recon_relax_kernel<grid, next forward, ...>.
    import re
    want = {"relax_bwd_lion_fwd": r"relax_bwd_lion_kernel<\d+, false, true,",
            "relax_bwd_lion": r"relax_bwd_lion_kernel<\d+, false, false,",
            "recon_bwd_lion_fwd": r"recon_relax_kernel<\d+, true,",
            "relax_fwd": r"relax_fwd_kernel<"}.get(call)
    if want is None:
        return None
    hits = [v for k, v in t.get("kernels", {}).items() if re.search(want, k)]
    return hits[0]["bytes_per_launch"] if len(hits) == 1 else None


def load_workload(name: str, dev):
    import numpy as np
    import torch
    import synthetic
    t0 = time.perf_counter()
    data = synthetic.generate(name, seed=0)
    wl = data["workload"]
    if wl.w_bf16:
        Wd = torch.from_numpy(data["W_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        Wd = torch.from_numpy(data["W"]).to(dev)
    Xd = torch.from_numpy(data["X_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    return data, Wd, Xd, time.perf_counter() - t0


def run_workload(name: str, args, dev, steps: int, warmup: int, headline: bool):
    """Set up one synthetic layer (or expert batch) and time ``steps`` fused
    steps after ``warmup`` untimed ones. Returns the measurement as a dict
    (the caller frees the device state)."""
    import numpy as np
    import torch
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver, tau_schedule

    data, Wd, Xd, gen_s = load_workload(name, dev)
    wl = data["workload"]
    lion = g.GsqLion.make(lr_logit=wl.lr_logit, lr_scale=1e-5)
    torch.cuda.synchronize()
    t_setup = time.perf_counter()
    solver = LayerSolver(Wd, Xd, wl.grid, tok_offsets=data["tok_offsets"],
                         rows_per_expert=wl.rows_per_expert or None, seed=0, stream_id=0, lion=lion,
                         init=args.init if headline else "rtn",
                         fuse=True if (headline and args.fuse) else "auto")
    torch.cuda.synchronize()
    setup_ms = (time.perf_counter() - t_setup) * 1e3
    M, K, N = solver.rows, solver.cols, solver.tokens
    coords = M * K
    bpc = bytes_per_coord(wl.grid, wl.w_bf16)

    if headline:
        # A plain copy of known size, untimed: its counter readings calibrate
        # FETCH_SIZE / WRITE_SIZE in the profiler runs (write_traffic).
        cal_src = torch.zeros(64 << 20, dtype=torch.float32, device=dev)
        cal_dst = torch.empty_like(cal_src)
        torch.neg(cal_src, out=cal_dst)
        del cal_src, cal_dst

    taus = tau_schedule(warmup + steps + 1)
    stream = torch.cuda.current_stream()
    # two products of 2*n_e*rows_e*K flops per expert (N = padded token total)
    rpe = solver.rows_per_expert
    gemm_flops = 4.0 * rpe * K * float(N)
    unfused = headline and args.unfused
    separate = None
    if unfused:
        solver.fuse = False
        start = solver.state()
        spin_up(lambda: solver.step(0, taus[0]))
        solver.load_state(start)
        del start
        for t in range(warmup):
            solver.step(t, taus[t])
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            t = warmup + i
            e = ev[i]
            e[0].record(stream)
            solver.relax_fwd(t, taus[t])
            e[1].record(stream)
            solver.recon()
            e[2].record(stream)
            solver.relax_bwd_lion(t, taus[t])
            e[3].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        rec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
        kernels = {
            "relax_fwd": {"ms": fwd_ms, "GB/s": bpc["fwd"] * coords / fwd_ms / 1e6},
            "recon_loss_grad": {"ms": rec_ms, "TFLOP/s": gemm_flops / rec_ms / 1e9},
            "relax_bwd_lion": {"ms": bwd_ms, "GB/s": bpc["bwd"] * coords / bwd_ms / 1e6},
        }
        relax_call, relax_ms = "relax_bwd_lion", fwd_ms + bwd_ms
        moved = bpc["fwd"] + bpc["bwd"]
    elif solver.fuse:
        elapsed, rec1_ms, fus_ms = time_fused(solver, taus, warmup, steps, stream)
        moved = bpc["fused"] - 4                     # no G read
        kernels = {
            "recon_residual": {"ms": rec1_ms, "TFLOP/s": gemm_flops / 2 / rec1_ms / 1e9,
                               "note": "first product R^T = dW X^T (2NMK flops; one grouped "
                                       "launch for an expert batch) and the loss partials"},
            "recon_bwd_lion_fwd": {"ms": fus_ms, "GB/s": moved * coords / fus_ms / 1e6,
                                   "TFLOP/s": gemm_flops / 2 / fus_ms / 1e9,
                                   "note": "second product G = 2 R^T X formed tile by tile and "
                                           "consumed by backward + Lion of step t and forward of "
                                           "step t+1 (G never stored; bytes moved)"},
        }
        relax_call, relax_ms = "recon_bwd_lion_fwd", fus_ms
        rec_ms = rec1_ms
    else:
        elapsed, rec_ms, fus_ms = time_fused(solver, taus, warmup, steps, stream)
        kernels = {
            "recon_loss_grad": {"ms": rec_ms, "TFLOP/s": gemm_flops / rec_ms / 1e9,
                                "note": "two bf16 GEMMs (2NMK flops each; one grouped launch "
                                        "each for an expert batch); the second sums the loss"},
            "relax_bwd_lion_fwd": {"ms": fus_ms, "GB/s": bpc["fused"] * coords / fus_ms / 1e6,
                                   "note": "backward + Lion of step t and forward of step t+1 "
                                           "(bytes moved)"},
        }
        relax_call, relax_ms = "relax_bwd_lion_fwd", fus_ms
        moved = bpc["fused"]
    if headline and not unfused and not args.no_ab:
        # The other form of the same step, for the A/B: with the second
        # product fused into the backward (G never stored), or with the
        # separate calls.
        fused = solver.fuse
        solver.fuse = not fused
        a_el, a_first, a_second = time_fused(solver, taus, min(warmup, 3), min(steps, 10), stream)
        solver.fuse = fused
        n_ab = min(steps, 10)
        separate = ({"ms_per_step": a_el * 1e3 / n_ab, "recon_loss_grad_ms": a_first,
                     "relax_bwd_lion_fwd_ms": a_second,
                     "note": "the same step with G stored by the second product and read back "
                             "by the relax pass"} if fused else
                    {"ms_per_step": a_el * 1e3 / n_ab, "recon_residual_ms": a_first,
                     "recon_bwd_lion_fwd_ms": a_second,
                     "note": "the same step with the second product fused into backward + Lion "
                             "+ next forward (gsq_recon_bwd_lion_fwd: G never stored)"})
    ms_per_step = elapsed * 1e3 / steps
    # Roofline of the relax work: the algorithmic bytes of one step's
    # forward + backward + Lion (the method's per-coordinate figure) over the
    # time of the kernel(s) that do it; beside it, the bytes the kernel moves.
    ach = bpc["step"] * coords / relax_ms / 1e6
    ach_moved = moved * coords / relax_ms / 1e6
    kname = {"recon_bwd_lion_fwd": "recon_relax_kernel (second product + backward + Lion + "
                                   "next forward)",
             "relax_bwd_lion_fwd": "relax_bwd_lion_kernel (fused backward + Lion + next forward)",
             "relax_bwd_lion": "relax_fwd_kernel + relax_bwd_lion_kernel"}[relax_call]
    roof = {"bound": "hbm", "kernel": kname,
            "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
            "traffic": measured_kernel_traffic(name, relax_call) if not unfused else None,
            "algorithmic_bytes_per_coord": bpc["step"],
            "algorithmic_bytes_per_launch": bpc["step"] * coords,
            "moved_bytes_per_coord": moved, "achieved_moved": ach_moved,
            "frac_moved": ach_moved / HBM_PEAK_GBS, "launch_ms": relax_ms}
    gflops = gemm_flops / 2 if solver.fuse else gemm_flops     # the separate products' flops
    gemm = {"achieved": gflops / rec_ms / 1e9, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": gflops / rec_ms / 1e9 / BF16_PEAK_TFLOPS,
            "products": "first only (the second runs inside the fused kernel)" if solver.fuse
            else "both"}
    res = {"name": wl.name, "workload": describe(wl), "value": coords * steps / elapsed,
           "ms_per_step": ms_per_step, "steps": steps, "warmup": warmup, "coords": coords,
           "rows": M, "cols": K, "tokens": int(data["tok_offsets"][-1]), "experts": wl.experts,
           "grid": ["int2", "ternary", "int3_local", "int3"][wl.grid], "lion_lr": wl.lr_logit,
           "roofline": roof, "recon_mfma": gemm, "kernels": kernels, "fused_product": solver.fuse,
           "last_loss": float(solver.loss.item()),
           "setup": {"init": args.init if headline else "rtn", "ms": setup_ms,
                     "inputs_drawn_s": gen_s,
                     "note": "warm start, X^T and state allocation, once per layer, not in the step"}}
    if separate is not None:
        res["ab_other_path"] = separate
    del solver
    torch.cuda.empty_cache()
    if wl.experts == 1 and not unfused and 2 * N > K:
        # The same step with the objective in Gram form (H = X^T X formed
        # once, untimed; one product of 2*M*K*K flops per step instead of two
        # of 2*N*M*K, fewer flops when N > K/2), on a fresh solver.
        gsol = LayerSolver(Wd, Xd, wl.grid, seed=0, stream_id=0, recon="gram", lion=lion)
        g_el, g_rec, g_fus = time_fused(gsol, taus, warmup, steps, stream)
        gram_flops = 2.0 * M * K * K
        res["gram"] = {
            "value": coords * steps / g_el, "unit": "weights/s", "ms_per_step": g_el * 1e3 / steps,
            "recon_gram": {"ms": g_rec, "TFLOP/s": gram_flops / g_rec / 1e9,
                           "note": "one bf16 GEMM dW H (2MK^2 flops) + loss finalize"},
            "relax_bwd_lion_fwd": {"ms": g_fus, "GB/s": bpc["fused"] * coords / g_fus / 1e6},
            "last_loss": float(gsol.loss.item())}
        del gsol
        torch.cuda.empty_cache()
    if name == "qproj4096_int2" and not unfused:
        # The two-product solve captured as one HIP graph.
        csol = LayerSolver(Wd, Xd, wl.grid, seed=0, stream_id=0, lion=lion)
        graph = csol.capture_solve(steps)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        c_el = (time.perf_counter() - t0) / 3
        res["graph"] = {"value": coords * steps / c_el, "unit": "weights/s",
                        "ms_per_step": c_el * 1e3 / steps,
                        "note": "the two-product step, whole solve replayed as one HIP graph"}
        del csol, graph
    del Wd, Xd
    torch.cuda.empty_cache()
    return res, data


def gemm_vs_vendor(I: int, J: int, K: int, dev, steps: int, warmup: int):
    """The plain bf16 NT product on seeded N(0,1) operands: this library's
    kernel and torch's matmul (hipBLASLt on ROCm) alternately, ``steps``
    timed calls each after ``warmup``, HIP events on the current stream.
    Prints one JSON line; the two outputs are compared (max relative
    difference) so the comparison is between products of the same result."""
    import torch
    import post_weight_quantization_philox_amd as g
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    A = torch.randn(I, K, device=dev, generator=gen).to(torch.bfloat16)
    B = torch.randn(J, K, device=dev, generator=gen).to(torch.bfloat16)
    C = torch.empty(I, J, device=dev, dtype=torch.bfloat16)
    C2 = torch.empty(I, J, device=dev, dtype=torch.bfloat16)
    Bt = B.t()
    ours = lambda: g.gsq_matmul_nt_bf16(I, J, K, A, K, B, K, C, J)
    vendor = lambda: torch.matmul(A, Bt, out=C2)
    res = {}
    for rep in range(2):
        for name, f in (("ours", ours), ("hipblaslt", vendor)):
            for _ in range(warmup):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                f()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            if rep == 1:
                res[name] = {"us": us, "TFLOP/s": 2.0 * I * J * K / us / 1e6}
    d = (C.float() - C2.float()).abs().max().item() / max(C2.float().abs().max().item(), 1e-30)
    print(json.dumps({"shape": [I, J, K], "steps": steps, **res, "max_rel_diff": d}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="dense headline: rows of the oracle sample (default: about 1.4e11 flops "
                         "of products)")
    ap.add_argument("--cpu-experts", type=int, default=2,
                    help="expert-batch headline: whole experts in the oracle sample (default 2)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="headline layer: moe64x2048x7168_int2 (default), qproj4096_int2, "
                         "downproj4096x14336_ternary, gateproj28672x8192_int3local, "
                         "gateproj28672x8192_int3full, linear512_int2")
    ap.add_argument("--block", action="store_true",
                    help="time GSQ's staged schedule over one Llama-3.1-8B-shaped decoder block "
                         "(random weights, 4096 tokens) instead of the per-layer step")
    ap.add_argument("--block-steps", type=int, default=50)
    ap.add_argument("--block-recon", default="auto", choices=("direct", "gram", "auto"),
                    help="reconstruction form per layer in --block: the two direct products, "
                         "the Gram form, or whichever needs fewer flops (default)")
    ap.add_argument("--block-objective", default="block", choices=("block", "layer"),
                    help="in --block: fit the output and down projections to the full-precision "
                         "block (default) or every layer to its own output")
    ap.add_argument("--init", choices=("rtn", "gptq"), default="rtn",
                    help="warm start of the headline layer; GPTQ's set-up time is reported "
                         "under 'setup' (not in the step)")
    ap.add_argument("--unfused", action="store_true",
                    help="time separate forward and backward calls instead of the fused pass")
    ap.add_argument("--no-variants", action="store_true",
                    help="measure the headline workload only")
    ap.add_argument("--fuse", action="store_true",
                    help="headline step with the second product fused into backward + Lion "
                         "(gsq_recon_bwd_lion_fwd) instead of the separate calls")
    ap.add_argument("--no-ab", action="store_true",
                    help="skip timing the other form of the headline step (fused / separate)")
    ap.add_argument("--gemm-vs-vendor", nargs=3, type=int, metavar=("I", "J", "K"),
                    help="time the plain bf16 NT product C = A B^T (I x K times J x K) with this "
                         "library's kernel and with torch's matmul (hipBLASLt) in one process, "
                         "for side-by-side profiles, and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 counter runs of this script into "
                         "profiles/traffic_<workload>.json and exit")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(args.workload, *args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the step shards by output rows with no "
              f"communication, so --gpus {args.gpus} is not run here", file=sys.stderr)
        sys.exit(2)

    import torch
    import post_weight_quantization_philox_amd as g

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    g.lib()
    dev = torch.device("cuda:0")
    if args.block:
        block_bench(args, dev)
        return
    if args.gemm_vs_vendor:
        gemm_vs_vendor(*args.gemm_vs_vendor, dev, args.steps, args.warmup)
        return
    head, data = run_workload(args.workload, args, dev, args.steps, args.warmup, headline=True)
    wl = data["workload"]
    cpu = None
    if not args.no_cpu_baseline:
        if wl.experts > 1:
            cpu = cpu_baseline(data, experts=max(1, min(args.cpu_experts, wl.experts)))
        else:
            M, K, N = wl.rows, wl.cols, int(data["tok_offsets"][-1])
            rows = args.cpu_rows or max(64, min(M, int(4096 * 4096 * 4096 // (K * N)) // 64 * 64))
            cpu = cpu_baseline(data, rows=rows)
    del data
    out = {
        "metric": "GSQ relax step weights/sec (fwd+recon+bwd+Lion)",
        "value": head["value"],
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "f32 relax+Lion, bf16 MFMA (fp32 accumulate)",
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "name", "rows", "cols", "tokens", "experts",
                                        "grid", "lion_lr")},
        "roofline": head["roofline"],
        "recon_mfma": head["recon_mfma"],
        "kernels": head["kernels"],
        "fused_product": head["fused_product"],
        "last_loss": head["last_loss"],
        "setup": head["setup"],
    }
    if "ab_other_path" in head:
        out["ab_other_path"] = head["ab_other_path"]
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if not args.no_variants:
        out["variants"] = {}
        for name in VARIANTS:
            if name == args.workload:
                continue
            res, _ = run_workload(name, args, dev, min(args.steps, 20), min(args.warmup, 5),
                                  headline=False)
            out["variants"][name] = res
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
