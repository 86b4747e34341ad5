"""Throughput of the GSQ relaxed-quantization step on one MI355X.

A step is one pass of the whole hot path over the layer: relaxed forward
(soft weights, dW), reconstruction loss and gradient (two bf16 MFMA
products), relaxed backward with the fused Lion update. The workload is a
Llama-3.1-8B-shaped q_proj: W 4096x4096 bf16 ~N(0, 0.02^2), 2-bit grid with
four fp32 logits per weight, group-128 scales, 4096 calibration tokens of
bf16 N(0,1) activations with 1 % outlier channels x20, Lion lr 1e-3.

Prints one JSON line: weights/s over the timed steps, per-call times from HIP
events recorded on the launch stream, the roofline of the dominant kernel,
and the CPU oracle's rate on a bounded sample of the same workload.
``--workload`` times one of the other synthetic layers instead (ternary
down_proj, 3-bit local-shift gate_proj, the 64-expert batch, the 512x512
layer); the default is the q_proj layer above.
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
WORKLOAD = "qproj4096_int2"
N_LOGITS = {0: 4, 1: 2, 2: 5, 3: 8}    # 2-bit, ternary, 3-bit local shift, full 3-bit


def bytes_per_coord(grid: int, w_bf16: bool) -> dict:
    """Algorithmic bytes per weight coordinate per call. Forward: L fp32
    logits + W read, dW (bf16) written. Backward + Lion: G, L logits and L
    momenta read, L logits and L momenta written. The fused backward + next
    forward adds W and dW. Local shift also reads its 1-byte warm-start code
    (once in the fused pass). Group scale traffic (< 0.2 B) is left out.
    2-bit bf16: 20 / 68 / 72 B."""
    L = N_LOGITS[grid]
    wb = 2 if w_bf16 else 4
    code = 1 if grid == 2 else 0
    return {"fwd": 4 * L + wb + 2 + code, "bwd": 4 + 16 * L + code,
            "fused": 4 + 16 * L + wb + 2 + code}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


# The sources the relax kernels (the dominant kernel's family) are built from.
RELAX_SOURCES = ("gsq_device.hpp", "gsq_internal.hpp", "relax.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "post_weight_quantization_philox_amd", "csrc")
    for fn in RELAX_SOURCES:
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel sources."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


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


def cpu_baseline(data, rows: int):
    """The oracle (NumPy fp64) on the first ``rows`` rows of a dense layer:
    one full step (relaxed forward, both products against all tokens,
    backward, Lion on logits and scales)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:            # threadpoolctl missing: report one thread
        blas_threads = 1
    wl = data["workload"]
    W = data["W"][:rows]
    X = data["X"]
    scales, codes, logits = oracle.init_rtn(W, wl.grid)
    state = {"logits": logits, "mom": np.zeros_like(logits), "scales": scales,
             "scale_mom": np.zeros_like(scales), "codes": codes}
    t0 = time.perf_counter()
    oracle.step(state, W, X, wl.grid, 0, 1.0, 0, 0, 1e-3, 1e-5, bf16_dW=True)
    dt = time.perf_counter() - t0
    return {"value": rows * W.shape[1] / dt, "unit": "weights/s", "cores": blas_threads,
            "kind": "oracle", "host": host_info(),
            "sample": f"one full step on rows 0..{rows - 1} of the {wl.rows}x{wl.cols} layer "
                      f"({rows * W.shape[1]} weights) against all {X.shape[0]} tokens, {dt:.1f} s; "
                      f"NumPy elementwise work on one thread, BLAS on {blas_threads}"}


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
    """Fused-step timing loop: returns (elapsed s, mean recon ms, mean fused
    backward+forward ms). Step t = objective of step t (dW from the previous
    pass) + backward and Lion of step t fused with the forward of step t + 1."""
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
        solver.recon()
        e[1].record(stream)
        solver.relax_bwd_lion_fwd(t, taus[t], t + 1, taus[t + 1])
        e[2].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    rec_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    fus_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    return elapsed, rec_ms, fus_ms


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
    staged_quantize(cfg, w, x[:256], g.GRID_INT2, 2, lion, recon=args.block_recon)   # warm up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, info = staged_quantize(cfg, w, x, g.GRID_INT2, args.block_steps, lion,
                              recon=args.block_recon)
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
                   "weights": n_w, "recon": args.block_recon},
        "stages": {k: {"seconds": v["seconds"], "recon": v["recon"]} for k, v in info.items()},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the oracle sample (default: about 1.4e11 flops of products)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="synthetic layer: linear512_int2, qproj4096_int2 (default), "
                         "downproj4096x14336_ternary, gateproj28672x8192_int3local, "
                         "gateproj28672x8192_int3full, moe64x2048x7168_int2")
    ap.add_argument("--block", action="store_true",
                    help="time GSQ's staged schedule over one Llama-3.1-8B-shaped decoder block "
                         "(random weights, 4096 tokens) instead of the per-layer step")
    ap.add_argument("--block-steps", type=int, default=50)
    ap.add_argument("--block-recon", default="auto", choices=("direct", "gram", "auto"),
                    help="reconstruction form per layer in --block: the two direct products, "
                         "the Gram form, or whichever needs fewer flops (default)")
    ap.add_argument("--init", choices=("rtn", "gptq"), default="rtn",
                    help="warm start; GPTQ's set-up time is reported under 'setup' (not in the step)")
    ap.add_argument("--unfused", action="store_true",
                    help="time separate forward and backward calls instead of the fused pass")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the Gram-form variant measured after the headline step")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the step shards by output rows with no "
              f"communication, so --gpus {args.gpus} is not run here", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synthetic
    import post_weight_quantization_philox_amd as g
    from post_weight_quantization_philox_amd.solver import LayerSolver, tau_schedule

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    g.lib()
    dev = torch.device("cuda:0")
    if args.block:
        block_bench(args, dev)
        return
    data = synthetic.generate(args.workload, seed=0)
    wl = data["workload"]
    if wl.w_bf16:
        Wd = torch.from_numpy(data["W_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        Wd = torch.from_numpy(data["W"]).to(dev)
    Xd = torch.from_numpy(data["X_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    lion = g.GsqLion.make(lr_logit=wl.lr_logit, lr_scale=1e-5)
    torch.cuda.synchronize()
    t_setup = time.perf_counter()
    solver = LayerSolver(Wd, Xd, wl.grid, tok_offsets=data["tok_offsets"],
                         rows_per_expert=wl.rows_per_expert or None, seed=0, stream_id=0, lion=lion,
                         init=args.init)
    torch.cuda.synchronize()
    setup_ms = (time.perf_counter() - t_setup) * 1e3
    M, K, N = solver.rows, solver.cols, solver.tokens
    coords = M * K
    bpc = bytes_per_coord(wl.grid, wl.w_bf16)
    FWD_BYTES_PER_COORD, BWD_BYTES_PER_COORD, FUSED_BYTES_PER_COORD = bpc["fwd"], bpc["bwd"], bpc["fused"]

    # A plain copy of known size, untimed: its counter readings calibrate
    # FETCH_SIZE / WRITE_SIZE in the profiler runs.
    cal_src = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)

    taus = tau_schedule(args.warmup + args.steps + 1)
    stream = torch.cuda.current_stream()
    # two products of 2*n_e*rows_e*K flops per expert (N = padded token total)
    rpe = solver.rows_per_expert
    gemm_flops = 4.0 * rpe * K * float(N)
    offs = [int(o) for o in solver.tok_offsets]
    n_gemm = 2 * max(1, sum(1 for e in range(len(offs) - 1) if offs[e + 1] > offs[e]))
    if args.unfused:
        spin_up(lambda: solver.step(0, taus[0]))
        for t in range(args.warmup):
            solver.step(t, taus[t])
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            t = args.warmup + i
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
            "relax_fwd": {"ms": fwd_ms, "GB/s": FWD_BYTES_PER_COORD * coords / fwd_ms / 1e6},
            "recon_loss_grad": {"ms": rec_ms, "TFLOP/s": gemm_flops / rec_ms / 1e9,
                                "note": "two bf16 GEMMs (2NMK flops each); GEMM2's first workgroup sums the loss"},
            "relax_bwd_lion": {"ms": bwd_ms, "GB/s": BWD_BYTES_PER_COORD * coords / bwd_ms / 1e6},
        }
        per_launch = {"relax_fwd": fwd_ms, "recon_loss_grad": rec_ms / n_gemm,
                      "relax_bwd_lion": bwd_ms}
        bytes_per = {"relax_fwd": FWD_BYTES_PER_COORD, "relax_bwd_lion": BWD_BYTES_PER_COORD}
    else:
        elapsed, rec_ms, fus_ms = time_fused(solver, taus, args.warmup, args.steps, stream)
        kernels = {
            "recon_loss_grad": {"ms": rec_ms, "TFLOP/s": gemm_flops / rec_ms / 1e9,
                                "note": "two bf16 GEMMs (2NMK flops each); GEMM2's first workgroup sums the loss"},
            "relax_bwd_lion_fwd": {"ms": fus_ms,
                                   "GB/s": FUSED_BYTES_PER_COORD * coords / fus_ms / 1e6,
                                   "note": "backward + Lion of step t and forward of step t+1"},
        }
        per_launch = {"recon_loss_grad": rec_ms / n_gemm, "relax_bwd_lion_fwd": fus_ms}
        bytes_per = {"relax_bwd_lion_fwd": FUSED_BYTES_PER_COORD}
    loss = float(solver.loss.item())
    ms_per_step = elapsed * 1e3 / args.steps

    # Dominant single kernel: the recon call is two products of equal flops
    # (each one launch, or two when its last round is split into 256x128
    # tiles), so each product is weighed at its share of the call.
    dominant = max(per_launch, key=per_launch.get)
    if dominant == "recon_loss_grad":
        ach = kernels[dominant]["TFLOP/s"]
        roof = {"bound": "mfma", "kernel": "gemm_nt_kernel (both products of the call)",
                "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / BF16_PEAK_TFLOPS, "traffic": None}
    else:
        per = bytes_per[dominant]
        ach = kernels[dominant]["GB/s"]
        roof = {"bound": "hbm", "kernel": dominant + "_kernel", "achieved": ach,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": measured_traffic(args.workload, dominant),
                "algorithmic_bytes_per_launch": per * coords}

    out = {
        "metric": "GSQ relax step weights/sec (fwd+recon+bwd+Lion)",
        "value": coords * args.steps / elapsed,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 relax+Lion, bf16 MFMA (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": describe(wl), "name": wl.name,
                   "rows": M, "cols": K, "tokens": int(data["tok_offsets"][-1]),
                   "experts": wl.experts, "grid": ["int2", "ternary", "int3_local", "int3"][wl.grid],
                   "lion_lr": wl.lr_logit},
        "roofline": roof,
        "kernels": kernels,
        "last_loss": loss,
        "setup": {"init": args.init, "ms": setup_ms,
                  "note": "warm start, X^T and state allocation, once per layer, not in the step"},
    }
    if not args.no_variants and not args.unfused and wl.experts == 1:
        # Same step with the objective in Gram form (H = X^T X formed once,
        # untimed; one product of 2*M*K*K flops per step instead of two of
        # 2*N*M*K), on a fresh solver. Reported beside the headline, which
        # keeps the two-product form.
        del solver
        torch.cuda.empty_cache()
        gsol = LayerSolver(Wd, Xd, wl.grid, seed=0, stream_id=0, recon="gram", lion=lion)
        g_el, g_rec, g_fus = time_fused(gsol, taus, args.warmup, args.steps, stream)
        gram_flops = 2.0 * M * K * K
        out["variants"] = {"gram": {
            "value": coords * args.steps / g_el, "unit": "weights/s",
            "ms_per_step": g_el * 1e3 / args.steps,
            "recon_gram": {"ms": g_rec, "TFLOP/s": gram_flops / g_rec / 1e9,
                           "note": "one bf16 GEMM dW H (2MK^2 flops) + loss finalize"},
            "relax_bwd_lion_fwd": {"ms": g_fus,
                                   "GB/s": FUSED_BYTES_PER_COORD * coords / g_fus / 1e6},
            "last_loss": float(gsol.loss.item()),
        }}
        del gsol
        # The same annealed steps captured as one HIP graph (launch overhead
        # removed; it matters for small layers), timed over one replay.
        torch.cuda.empty_cache()
        csol = LayerSolver(Wd, Xd, wl.grid, seed=0, stream_id=0, lion=lion)
        graph = csol.capture_solve(args.steps)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        g_el = (time.perf_counter() - t0) / 3
        out["variants"]["graph"] = {
            "value": coords * args.steps / g_el, "unit": "weights/s",
            "ms_per_step": g_el * 1e3 / args.steps,
            "note": "the two-product step, whole K-step solve replayed as one HIP graph"}
        del csol, graph
    if not args.no_cpu_baseline and wl.experts == 1:
        rows = args.cpu_rows or max(64, min(M, int(4096 * 4096 * 4096 // (K * N)) // 64 * 64))
        out["cpu_baseline"] = cpu_baseline(data, rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
