#!/usr/bin/env python3
"""Benchmark: one HQ-MM linear-layer step (forward Y, input gradient dX, weight gradient dW,
HALO-2 rotations, tensor-wise INT8) on one MI355X, through the C ABI of libhq.

A step is the whole hot path on one batch: rotate+quantize X, W and dY, the three INT8 MFMA
GEMMs with dequantization, and the output-side inverse rotations. Inputs are seeded synthetic
tensors with the workload's shapes and distributions, resident in HBM before timing starts.

Printed (one JSON line): effective TOPS = sum of 2*M*N*K over the three products / step
time of an uninstrumented timed region; the percentage of the INT8 MFMA peak; the roofline of
the dominant kernel (the GEMM, its launches stamped with HIP events on their own stream during
a second pass of the same steps); the rotate+quantize bandwidth; an unrotated bf16 GEMM
baseline of the same three products; the step of the Llama-7B-shaped layer against its bf16
baseline; and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_hbm_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "hadamard_rotated_precision_amd", "csrc", "hq_gemm.hip")


def gemm_source_hash():
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def layer_ops(cfg):
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    ops = 0
    if "fwd" in cfg["passes"]:
        ops += 2 * N * D * C
    if "dx" in cfg["passes"]:
        ops += 2 * N * C * D
    if "dw" in cfg["passes"]:
        ops += 2 * D * C * N
    return ops


def prologue_bytes(cfg, in_bytes):
    """Algorithmic bytes of the rotate+quantize stage of one step: each input read once, each
    code tensor the method defines written once (X: qX and, under HALO-2, qXt)."""
    from hadamard_rotated_precision_amd import workloads as WL
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    nx_codes = 2 if cfg["variant"] == WL.HALO2 else 1
    b = N * C * (in_bytes + nx_codes) + D * C * (in_bytes + 1)
    if "dx" in cfg["passes"] or "dw" in cfg["passes"]:
        b += N * D * (in_bytes + 1)
    return b


def cpu_baseline(cfg_id, tokens):
    """The oracle (plain C, OpenMP) on a bounded sample: the same workload with fewer tokens."""
    import oracle as O
    from hadamard_rotated_precision_amd import workloads as WL
    cfg = WL.config(cfg_id)
    k = cfg["k"]
    tokens = max(k, tokens // k * k)
    cfg = WL.config(cfg_id, N=tokens)
    inputs = WL.make_inputs(cfg)
    dt = cfg["in_dtype"]
    X = O.decode(inputs["x"], dt)
    W = O.decode(inputs["w"], dt)
    dY = O.decode(inputs["dy"], dt) if inputs.get("dy") is not None else None
    t0 = time.perf_counter()
    O.linear(X, W, dY, k, cfg["bits"], cfg["variant"], cfg["mode"], inputs.get("steps"),
             cfg["passes"])
    dt_s = time.perf_counter() - t0
    ops = layer_ops(cfg)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": ops / dt_s / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": "%s with N=%d tokens (same C, D, k, distributions): rotate, quantize, "
                      "int64 GEMMs, exact inverse rotations, dequantize for %s; %.2f s"
                      % (cfg["name"], tokens, "+".join(cfg["passes"]), dt_s),
            "seconds": dt_s}


def bf16_baseline(cfg, steps, warmup, library):
    """Three unrotated bf16 GEMMs of the same shapes (timing context only)."""
    import torch
    torch.backends.cuda.preferred_blas_library(library)
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((N, C), device="cuda", dtype=torch.bfloat16, generator=g)
    w = torch.randn((D, C), device="cuda", dtype=torch.bfloat16, generator=g)
    dy = torch.randn((N, D), device="cuda", dtype=torch.bfloat16, generator=g)

    def run():
        torch.mm(x, w.t())
        torch.mm(dy, w)
        torch.mm(dy.t(), x)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        run()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def fwht_bandwidth(reps=20, rows=8192, cols=13824, k=128):
    """hq_fwht on its own (bf16 in, bf16 out), RIGHT and LEFT, on the largest operand shape of
    the workloads (X of the 8192 x 13824 x 5120 layer, k = 128): algorithmic bytes = 2 B read
    + 2 B written per element, over the mean launch time (events on the launch stream)."""
    import torch
    from hadamard_rotated_precision_amd import binding as B
    from hadamard_rotated_precision_amd import tensors as T
    gen = torch.Generator(device="cuda")
    gen.manual_seed(106)
    src = torch.randn((rows, cols), dtype=torch.float32, device="cuda", generator=gen).to(torch.bfloat16)
    dst = torch.empty_like(src)
    res = {"shape": "%dx%d bf16 -> bf16" % (rows, cols), "k": k,
           "bytes_per_launch": 4 * rows * cols}
    for name, rot in (("right", B.HQ_ROT_RIGHT), ("left", B.HQ_ROT_LEFT)):
        def run():
            B.check(B.hq_fwht(src.data_ptr(), B.HQ_BF16, dst.data_ptr(), B.HQ_BF16, rows, cols,
                              rot, k, T.stream_ptr()), "fwht")
        for _ in range(3):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gbs = 4.0 * rows * cols / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "gbps": round(gbs, 1),
                     "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 1)}
    return res


def layer_vs_bf16(cfg_id, steps, warmup):
    """The HQ-MM step of another workload (inputs resident, no instrumentation) next to the
    three unrotated bf16 GEMMs of the same shapes: the comparison the target names for the
    Llama-7B-shaped MLP layer."""
    import torch
    from hadamard_rotated_precision_amd import tensors as T
    from hadamard_rotated_precision_amd import workloads as WL
    cfg = WL.config(cfg_id)
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    inputs = WL.make_inputs(cfg)
    dev = "cuda"
    in_dt, out_dt = cfg["in_dtype"], cfg["out_dtype"]
    x = T.device_tensor_from_bits(inputs["x"], in_dt, dev)
    w = T.device_tensor_from_bits(inputs["w"], in_dt, dev)
    dy = T.device_tensor_from_bits(inputs["dy"], in_dt, dev)
    layer = T.Layer(N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"], device=dev)
    odt = T.TORCH_DT[out_dt]
    y = torch.empty((N, D), dtype=odt, device=dev)
    dx = torch.empty((N, C), dtype=odt, device=dev)
    dw = torch.empty((D, C), dtype=odt, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        layer.fwd(x, w, y, None, stream)
        layer.bwd_input(dy, dx, None, stream)
        layer.bwd_weight(dw, stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del x, w, dy, y, dx, dw, layer
    ms_rb = bf16_baseline(cfg, steps, warmup, "cublas")
    ms_lt = bf16_baseline(cfg, steps, warmup, "cublaslt")
    return {"workload": cfg["name"], "hq_ms_per_step": round(ms, 4),
            "hq_tops": round(layer_ops(cfg) / (ms * 1e-3) / 1e12, 1),
            "bf16_ms_rocblas": round(ms_rb, 4), "bf16_ms_hipblaslt": round(ms_lt, 4),
            "speedup_vs_rocblas": round(ms_rb / ms, 3), "speedup_vs_hipblaslt": round(ms_lt / ms, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2,
                    help="workload id (default 2: HALO-2 step, 2048 x 4096 x 4096, k=256)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=512)
    ap.add_argument("--check-config", type=int, default=4,
                    help="also time this workload's step against three bf16 GEMMs (default 4: "
                         "the Llama-7B-shaped MLP layer); 0 to skip")
    ap.add_argument("--no-fwht", action="store_true",
                    help="skip the standalone hq_fwht bandwidth figure")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache prologue pass (kernel traces of the warm step)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB three times with a "
                         "plain device copy (reference dispatches for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from hadamard_rotated_precision_amd import binding as B
    from hadamard_rotated_precision_amd import tensors as T
    from hadamard_rotated_precision_amd import workloads as WL

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    B.load()
    cfg = WL.config(args.config)
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    in_dt, out_dt = cfg["in_dtype"], cfg["out_dtype"]
    print("[bench] workload %s: generating inputs" % cfg["name"], file=sys.stderr, flush=True)
    inputs = WL.make_inputs(cfg)
    dev = "cuda"
    x = T.device_tensor_from_bits(inputs["x"], in_dt, dev)
    w = T.device_tensor_from_bits(inputs["w"], in_dt, dev)
    has_bwd = "dx" in cfg["passes"] or "dw" in cfg["passes"]
    dy = T.device_tensor_from_bits(inputs["dy"], in_dt, dev) if has_bwd else None
    steps_t = None
    if cfg["mode"] == WL.STEP:
        steps_t = {n: torch.tensor([v], dtype=torch.float32, device=dev)
                   for n, v in inputs["steps"].items()}
    layer = T.Layer(N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"], device=dev)
    odt = T.TORCH_DT[out_dt]
    y = torch.empty((N, D), dtype=odt, device=dev)
    dx = torch.empty((N, C), dtype=odt, device=dev) if "dx" in cfg["passes"] else None
    dw = torch.empty((D, C), dtype=odt, device=dev) if "dw" in cfg["passes"] else None
    stream = torch.cuda.current_stream()

    def step():
        layer.fwd(x, w, y, steps_t, stream)
        if dx is not None:
            layer.bwd_input(dy, dx, steps_t, stream)
        if dw is not None:
            layer.bwd_weight(dw, stream)

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: 3 copies of %d bytes" % (4 * n), file=sys.stderr, flush=True)
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # ---- timed region: K steps, uninstrumented (per-launch events cost several us per launch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ops = layer_ops(cfg)
    eff_tops = ops / (ms_per_step * 1e-3) / 1e12
    print("[bench] timed region done: %.3f ms/step" % ms_per_step, file=sys.stderr, flush=True)

    # ---- roofline pass: the same K steps again, each GEMM launch stamped with HIP events on
    # its own launch stream (hipExtLaunchKernel records the kernel's start and end)
    B.check(B.hq_profile_start(1 << B.HQ_KIND_GEMM), "profile")
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    prof = B.profile_stop_dict()
    ms_instr = (t3 - t2) * 1e3 / args.steps
    gcount, gms, gunits = prof["gemm"]
    gemm_tops = gunits / (gms * 1e-3) / 1e12 if gms > 0 else None
    gemm_avg_us = gms * 1e3 / gcount if gcount else None

    # ---- per-kind breakdown of the same step (all kinds bracketed; a separate pass)
    B.check(B.hq_profile_start((1 << B.HQ_KIND_COUNT) - 1), "profile")
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    breakdown = B.profile_stop_dict()

    # ---- rotate+quantize bandwidth: the prologue launches alone
    in_bytes = 2 if in_dt != WL.F32 else 4
    pro_bytes = prologue_bytes(cfg, in_bytes)
    pro_ms = 0.0
    for kind in ("rot_absmax", "rot_quant", "transpose", "misc"):
        pro_ms += breakdown[kind][1]
    pro_ms_step = pro_ms / args.steps
    rq_gbs = pro_bytes / (pro_ms_step * 1e-3) / 1e9 if pro_ms_step > 0 else None

    # ---- the same with cold caches: before each step a 512 MB buffer is written, which evicts
    # the inputs from L2 and the 256 MB MALL, so the prologue reads them from HBM
    rq_cold = None
    pro_cold_ms = 0.0
    if not args.no_cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_steps = max(5, min(args.steps, 20))
        B.check(B.hq_profile_start((1 << B.HQ_KIND_ROT_ABSMAX) | (1 << B.HQ_KIND_ROT_QUANT)),
                "profile")
        for _ in range(cold_steps):
            flush.fill_(1)
            step()
        torch.cuda.synchronize()
        cold = B.profile_stop_dict()
        del flush
        pro_cold_ms = (cold["rot_absmax"][1] + cold["rot_quant"][1]) / cold_steps
    if pro_cold_ms > 0:
        gbs = pro_bytes / (pro_cold_ms * 1e-3) / 1e9
        rq_cold = {"ms_per_step": round(pro_cold_ms, 4), "gbps": round(gbs, 1),
                   "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 1),
                   "what": "prologue algorithmic bytes over the prologue kernels' event time, "
                           "a 512 MB buffer written before each of %d steps" % cold_steps}

    # counted bytes (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated) from profiles/, used only
    # while the sources they were taken from are unchanged
    traffic = None
    rq_counted = None
    if os.path.exists(TRAFFIC_FILE):
        from hadamard_rotated_precision_amd.prof_summary import prologue_source_hash
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("workload") == cfg["name"]:
            if tr.get("gemm_source_sha256_16") == gemm_source_hash():
                traffic = tr.get("bytes_per_launch")
            pb = tr.get("prologue_bytes_per_step")
            if pb and pro_ms_step > 0 and \
                    tr.get("prologue_source_sha256_16") == prologue_source_hash():
                gbs = pb / (pro_ms_step * 1e-3) / 1e9
                rq_counted = {"bytes_per_step": pb, "gbps": round(gbs, 1),
                              "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 1),
                              "source": "rocprofv3 FETCH_SIZE + WRITE_SIZE of every prologue "
                                        "dispatch, calibrated on a 1 GiB device copy "
                                        "(profiles/gemm_hbm_traffic.json)"}

    result = {
        "metric": "HQ-MM fwd+bwd effective TOPS and % of INT8 MFMA peak; rotate+quant GB/s",
        "value": round(eff_tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "N": N, "C": C, "D": D, "k": cfg["k"],
                   "bits": cfg["bits"], "variant": ["HALO0", "HQ", "HALO2"][cfg["variant"]],
                   "in_dtype": WL.DTYPE_NAMES[in_dt], "out_dtype": WL.DTYPE_NAMES[out_dt],
                   "passes": list(cfg["passes"]), "parallelism": "single GPU"},
        "pct_int8_peak": round(100.0 * eff_tops / PEAK_INT8_TOPS, 2),
        "gemm_tops": None if gemm_tops is None else round(gemm_tops, 1),
        "rotate_quant_gbps": None if rq_gbs is None else round(rq_gbs, 1),
        "rotate_quant_pct_hbm": None if rq_gbs is None else round(100 * rq_gbs / PEAK_HBM_GBS, 1),
        "rotate_quant_counted": rq_counted,
        "rotate_quant_cold": rq_cold,
        "roofline": {
            "kernel": "gemm_i8_kernel (int8 MFMA GEMM + dequant epilogue)",
            "bound": "mfma",
            "achieved": None if gemm_tops is None else round(gemm_tops, 1),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s",
            "frac": None if gemm_tops is None else round(gemm_tops / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "launches": gcount,
            "avg_launch_us": None if gemm_avg_us is None else round(gemm_avg_us, 2),
            "ops_per_launch": None if not gcount else gunits / gcount,
            "timing": "HIP events stamped by hipExtLaunchKernel on each GEMM launch, over a "
                      "second pass of the same %d steps (%.4f ms/step with the events)"
                      % (args.steps, ms_instr),
        },
        "breakdown_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in breakdown.items()},
    }
    if not args.no_bf16_baseline:
        try:
            ms_rb = bf16_baseline(cfg, args.steps, args.warmup, "cublas")
            ms_lt = bf16_baseline(cfg, args.steps, args.warmup, "cublaslt")
            result["bf16_baseline"] = {
                "what": "three unrotated bf16 torch.mm of the same shapes (Y, dX, dW)",
                "ms_rocblas": round(ms_rb, 4), "ms_hipblaslt": round(ms_lt, 4),
                "speedup_vs_rocblas": round(ms_rb / ms_per_step, 3),
                "speedup_vs_hipblaslt": round(ms_lt / ms_per_step, 3)}
        except Exception as exc:  # report, do not fail the benchmark line
            result["bf16_baseline"] = {"error": str(exc)}
    if args.check_config and args.check_config != args.config:
        print("[bench] step vs bf16 on config %d" % args.check_config, file=sys.stderr, flush=True)
        try:
            result["layer_vs_bf16"] = layer_vs_bf16(args.check_config, max(5, args.steps // 5),
                                                    max(2, args.warmup // 2))
        except Exception as exc:  # report, do not fail the benchmark line
            result["layer_vs_bf16"] = {"error": str(exc)}
    if not args.no_fwht:
        print("[bench] hq_fwht bandwidth", file=sys.stderr, flush=True)
        try:
            result["fwht"] = fwht_bandwidth()
        except Exception as exc:  # report, do not fail the benchmark line
            result["fwht"] = {"error": str(exc)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.config, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
