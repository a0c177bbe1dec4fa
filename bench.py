#!/usr/bin/env python3
"""Benchmark: one HQ-MM linear-layer step (forward Y, input gradient dX, weight gradient dW,
HALO-2 rotations, tensor-wise INT8) on one MI355X, through the C ABI of libhq.

A step is the whole hot path on one batch: rotate+quantize X, W and dY, the three INT8 MFMA
GEMMs with dequantization, and the output-side inverse rotations. Inputs are seeded synthetic
tensors with the workload's shapes and distributions, resident in HBM before timing starts.
The default workload is the largest one, the Qwen-14B-shaped down projection
(8192 x 13824 x 5120, k = 128, HALO-2, bf16).

Printed (one JSON line): effective TOPS = sum of 2*M*N*K over the three products / step
time of an uninstrumented timed region; the percentage of the INT8 MFMA peak; the roofline of
the dominant kernel (the GEMM, its launches stamped with HIP events on their own stream during
a second pass of the same steps, per product and overall); the rotate+quantize bandwidth; an
unrotated bf16 GEMM baseline of the same three products; the steps of the Llama-7B-shaped
layer and of the 2048 x 4096 x 4096 layer against their bf16 baselines; hq_fwht through the
butterfly and matrix-core paths; and the CPU oracle timed on a bounded sample of the same
workload.

Step comparisons against bf16 use one method on both sides: an event pair on the stream around
each step, 5 warm-up steps, then the median of 20.
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA, 5.0 PFLOP/s
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg_id, tokens):
    """The oracle (plain C, OpenMP over output rows) on a bounded sample: the same workload
    with fewer tokens (the weight tensor is still rotated and quantized whole)."""
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
    return {"value": ops / dt_s / 1e12, "unit": "TOPS", "cores": O.threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": "%s with N=%d tokens (same C, D, k, distributions; W rotated and "
                      "quantized whole): rotate, quantize, int64 GEMMs, exact inverse rotations, "
                      "dequantize for %s; %.2f s"
                      % (cfg["name"], tokens, "+".join(cfg["passes"]), dt_s),
            "seconds": dt_s}


def event_median_ms(fn, warmup=5, reps=20):
    """GPU time of fn() on the current stream: an event pair around each call, after `warmup`
    calls; the median of `reps` calls in ms."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    times = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return times[len(times) // 2]


def bf16_baseline(cfg, library):
    """Three unrotated bf16 GEMMs of the same shapes (timing context only): event median."""
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
    ms = event_median_ms(run)
    torch.backends.cuda.preferred_blas_library("default")
    return ms


def fwht_bandwidth(reps=20, rows=8192, cols=13824, ks=(16, 32, 64, 128, 256)):
    """hq_fwht on its own (bf16 in, bf16 out), RIGHT and LEFT, on the largest operand shape of
    the workloads (X of the 8192 x 13824 x 5120 layer), through the VALU butterflies and the
    matrix cores at each k: algorithmic bytes = 2 B read + 2 B written per element, over the
    mean launch time (events on the launch stream). `auto` names the path hq_fwht takes."""
    import torch
    from hadamard_rotated_precision_amd import binding as B
    from hadamard_rotated_precision_amd import tensors as T
    gen = torch.Generator(device="cuda")
    gen.manual_seed(106)
    src = torch.randn((rows, cols), dtype=torch.float32, device="cuda", generator=gen).to(torch.bfloat16)
    dst = torch.empty_like(src)
    res = {"shape": "%dx%d bf16 -> bf16" % (rows, cols), "bytes_per_launch": 4 * rows * cols}
    for name, rot in (("right", B.HQ_ROT_RIGHT), ("left", B.HQ_ROT_LEFT)):
        res[name] = {}
        for k in ks:
            row = {}
            for pname, path in (("butterfly", B.HQ_FWHT_BUTTERFLY), ("matrix", B.HQ_FWHT_MATRIX)):
                def run():
                    B.check(B.hq_fwht_path(src.data_ptr(), B.HQ_BF16, dst.data_ptr(), B.HQ_BF16,
                                           rows, cols, rot, k, path, T.stream_ptr()), "fwht")
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
                row[pname] = {"us": round(us, 2), "gbps": round(gbs, 1),
                              "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 1)}
            # hq_fwht's HQ_FWHT_AUTO choice, as its header states it (context for the reader)
            auto_matrix = rot == B.HQ_ROT_LEFT and k >= 256
            row["auto"] = "matrix" if auto_matrix else "butterfly"
            res[name]["k%d" % k] = row
    return res


def layer_vs_bf16(cfg_id):
    """The HQ-MM step of a workload (inputs resident, no instrumentation) next to the three
    unrotated bf16 GEMMs of the same shapes, both timed by event_median_ms: the comparison the
    target names for the Llama-7B-shaped MLP layer."""
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
    ms = event_median_ms(step)
    del x, w, dy, y, dx, dw, layer
    ms_rb = bf16_baseline(cfg, "cublas")
    ms_lt = bf16_baseline(cfg, "cublaslt")
    return {"workload": cfg["name"], "hq_ms_per_step": round(ms, 4),
            "hq_tops": round(layer_ops(cfg) / (ms * 1e-3) / 1e12, 1),
            "bf16_ms_rocblas": round(ms_rb, 4), "bf16_ms_hipblaslt": round(ms_lt, 4),
            "speedup_vs_rocblas": round(ms_rb / ms, 3), "speedup_vs_hipblaslt": round(ms_lt / ms, 3),
            "timing": "event pair around each step on the stream, 5 warm-ups, median of 20 "
                      "(the same for the bf16 GEMMs)"}


def fp8_step(cfg_id, steps=20, fmt=None):
    """The same layer step with float codes, FP8 E4M3 by default (HALO page: the FP8 and FP6
    variants of the three matmuls; FP6 codes, E2M3 or E3M2, are kept as E4M3 bytes and run on
    the same FP8 matrix-core product, as the page ran FP6 on FP8 hardware): step time by event
    median, and the GEMM's roofline against the 5.0 PFLOP/s dense FP8 peak (algorithmic
    2*M*N*K flops per launch over kernel-stamped launch times)."""
    import torch
    from hadamard_rotated_precision_amd import binding as B
    from hadamard_rotated_precision_amd import tensors as T
    from hadamard_rotated_precision_amd import workloads as WL
    fmt = WL.E4M3 if fmt is None else fmt
    cfg = WL.config(cfg_id, fmt=fmt)
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    inputs = WL.make_inputs(cfg)
    dev = "cuda"
    in_dt, out_dt = cfg["in_dtype"], cfg["out_dtype"]
    x = T.device_tensor_from_bits(inputs["x"], in_dt, dev)
    w = T.device_tensor_from_bits(inputs["w"], in_dt, dev)
    dy = T.device_tensor_from_bits(inputs["dy"], in_dt, dev)
    layer = T.Layer(N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"], device=dev,
                    fmt=fmt)
    odt = T.TORCH_DT[out_dt]
    y = torch.empty((N, D), dtype=odt, device=dev)
    dx = torch.empty((N, C), dtype=odt, device=dev)
    dw = torch.empty((D, C), dtype=odt, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        layer.fwd(x, w, y, None, stream)
        layer.bwd_input(dy, dx, None, stream)
        layer.bwd_weight(dw, stream)
    ms = event_median_ms(step)
    B.check(B.hq_profile_start(1 << B.HQ_KIND_GEMM), "profile")
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    _, gms, gunits = B.profile_stop_dict()["gemm"]
    tf = gunits / (gms * 1e-3) / 1e12
    return {"workload": cfg["name"], "ms_per_step": round(ms, 4),
            "tflops": round(layer_ops(cfg) / (ms * 1e-3) / 1e12, 1),
            "gemm_roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4)},
            "timing": "event median of 20 steps after 5 warm-ups; GEMM launches stamped by "
                      "hipExtLaunchKernel over %d further steps" % steps}


def bmm_step(steps=20):
    """The batched HQ-MM of attention scores (INT4 page §A.1): S = Q K^T with its two
    gradients for a Llama-7B-shaped attention layer (4 x 32 heads, 1024 tokens, head_dim 128,
    k = 128, HALO-2, bf16): step time by event median, effective TOPS and the GEMM roofline."""
    import torch
    from hadamard_rotated_precision_amd import binding as B
    from hadamard_rotated_precision_amd import tensors as T
    from hadamard_rotated_precision_amd import workloads as WL
    cfg = WL.attention_config()
    nb, N, C, D = cfg["batch"], cfg["N"], cfg["C"], cfg["D"]
    inputs = WL.make_batched_inputs(cfg)
    dt = cfg["in_dtype"]
    x = T.device_tensor_from_bits(inputs["x"], dt)
    w = T.device_tensor_from_bits(inputs["w"], dt)
    dy = T.device_tensor_from_bits(inputs["dy"], dt)
    L = T.BatchedLayer(nb, N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"])
    odt = T.TORCH_DT[cfg["out_dtype"]]
    y = torch.empty((nb, N, D), dtype=odt, device="cuda")
    dx = torch.empty((nb, N, C), dtype=odt, device="cuda")
    dw = torch.empty((nb, D, C), dtype=odt, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        L.fwd(x, w, y, None, stream)
        L.bwd_input(dy, dx, None, stream)
        L.bwd_weight(dw, stream)
    ms = event_median_ms(step)
    B.check(B.hq_profile_start(1 << B.HQ_KIND_GEMM), "profile")
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    _, gms, gunits = B.profile_stop_dict()["gemm"]
    tops = gunits / (gms * 1e-3) / 1e12
    ops = 3 * 2 * nb * N * C * D
    return {"workload": cfg["name"], "ms_per_step": round(ms, 4),
            "tops": round(ops / (ms * 1e-3) / 1e12, 1),
            "gemm_roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": PEAK_INT8_TOPS,
                              "unit": "TOP/s", "frac": round(tops / PEAK_INT8_TOPS, 4)}}


def lss_step(cfg_id, reps=20):
    """LSS-MM (INT4 page §4.2, §A.3, §A.6) on a workload's shapes, distributions and k as an
    INT4 HQ layer (X codes from an absmax INT4 HQ forward): the sampled weight gradient at
    budget N/2 next to the unsampled INT4 weight gradient of the same layer (event medians),
    with each stage's launch time (kernel-stamped events over `reps` calls), its algorithmic
    bytes and GB/s, and the GEMM's ops over the kept tokens."""
    import torch
    from hadamard_rotated_precision_amd import binding as B
    from hadamard_rotated_precision_amd import tensors as T
    from hadamard_rotated_precision_amd import workloads as WL
    cfg = WL.config(cfg_id)
    N, C, D, k = cfg["N"], cfg["C"], cfg["D"], cfg["k"]
    inputs = WL.make_inputs(cfg)
    dt = cfg["in_dtype"]
    x = T.device_tensor_from_bits(inputs["x"], dt)
    w = T.device_tensor_from_bits(inputs["w"], dt)
    dy = T.device_tensor_from_bits(inputs["dy"], dt)
    layer = T.Layer(N, C, D, k, 4, WL.ABSMAX, WL.HQ)
    odt = T.TORCH_DT[cfg["out_dtype"]]
    y = torch.empty((N, D), dtype=odt, device="cuda")
    dx = torch.empty((N, C), dtype=odt, device="cuda")
    dw_full = torch.empty((D, C), dtype=odt, device="cuda")
    dw = torch.empty((D, C), dtype=odt, device="cuda")
    layer.fwd(x, w, y)
    layer.bwd_input(dy, dx)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg["seed"] + 7)
    u = torch.rand(N, generator=gen, device="cuda", dtype=torch.float32)
    lss = T.LssGrad(N, C, D, k)
    budget = N / 2
    full_ms = event_median_ms(lambda: layer.bwd_weight(dw_full))
    lss_ms = event_median_ms(lambda: lss(dy, layer.qx, u, dw, budget))
    B.check(B.hq_profile_start((1 << B.HQ_KIND_COUNT) - 1), "profile")
    for _ in range(reps):
        lss(dy, layer.qx, u, dw, budget)
    torch.cuda.synchronize()
    B.profile_stop_dict()
    recs = B.profile_records()
    kept = lss.read_stats()[0]
    kpad = (kept + 15) // 16 * 16
    eb = 4 if dt == WL.F32 else 2
    names = ["rowmax", "score", "prob", "pack", "gemm"]
    nbytes = {"rowmax": N * D * eb + N * 4,
              "score": N * D * eb + N * C + N * 8,
              "prob": N * (8 + 4 + 4 + 8 + 1) + kept * 4,
              "pack": kept * (D * eb + C + 4 + 8) + (D + C) * kpad,
              "gemm": (D + C) * kpad + D * C * eb}
    stages = {}
    per = len(recs) // reps   # four sampling stages, then the GEMM's launch(es)
    if per >= len(names) and len(recs) == per * reps:
        for i, nm in enumerate(names):
            idx = [i] if nm != "gemm" else list(range(len(names) - 1, per))
            ms = sorted(sum(recs[j * per + q][1] for q in idx) for j in range(reps))[reps // 2]
            st = {"us": round(ms * 1e3, 2), "bytes": nbytes[nm],
                  "gbps": round(nbytes[nm] / (ms * 1e-3) / 1e9, 1)}
            if nm == "gemm":
                st["launches"] = len(idx)
            if nm == "gemm":
                tops = 2.0 * C * D * kept / (ms * 1e-3) / 1e12
                st["tops"] = round(tops, 1)
                st["frac_int8_peak"] = round(tops / PEAK_INT8_TOPS, 4)
            stages[nm] = st
    return {"workload": "lss_int4_%dx%dx%d_k%d_from_%s" % (N, C, D, k, cfg["name"]), "budget": budget,
            "kept": kept, "lss_ms": round(lss_ms, 4), "unsampled_int4_dw_ms": round(full_ms, 4),
            "speedup_vs_unsampled": round(full_ms / lss_ms, 3), "stages_median": stages,
            "timing": "event median of 20 calls after 5 warm-ups for both; stages: median of "
                      "%d kernel-stamped launches each" % reps}


def qparam_stats(reps=10):
    """Quantizer-parameter statistics (INT4 page §A.3-§A.5) on X of the 8192 x 13824 x 5120
    layer (bf16, k = 128): the LSQ step gradient (reads X and a gradient of the same shape,
    2 x 226 MB), the cold-start step and the quantization error (X only), each one streaming
    pass: GB/s over the mean event time; and hq_select_hadamard_k over k = 16..256 for that
    layer's X and W (a synchronous setup call: wall time)."""
    import ctypes
    import torch
    from hadamard_rotated_precision_amd import binding as B
    from hadamard_rotated_precision_amd import tensors as T
    rows, cols, k, D = 8192, 13824, 128, 5120
    gen = torch.Generator(device="cuda")
    gen.manual_seed(107)
    x = torch.randn((rows, cols), dtype=torch.float32, device="cuda", generator=gen).to(torch.bfloat16)
    g = (torch.randn((rows, cols), dtype=torch.float32, device="cuda", generator=gen) * 1e-3).to(torch.bfloat16)
    w = (torch.randn((D, cols), dtype=torch.float32, device="cuda", generator=gen) * 0.015).to(torch.bfloat16)
    cfg = T.config(k, 8, B.HQ_SCALE_ABSMAX, B.HQ_VARIANT_HQ)
    nws = B.hq_workspace_bytes(cfg, 1, 16, 1)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    sc = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    out = torch.zeros(1, dtype=torch.float64, device="cuda")
    step = torch.zeros(1, dtype=torch.float32, device="cuda")
    res = {"shape": "%dx%d bf16, k=%d" % (rows, cols, k)}

    def timed(fn, nbytes):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us": round(us, 2), "gbps": round(gbs, 1), "pct_hbm": round(100 * gbs / PEAK_HBM_GBS, 1)}
    n2 = 2 * rows * cols
    res["lsq_grad"] = timed(lambda: B.check(B.hq_rotated_stat(
        x.data_ptr(), g.data_ptr(), B.HQ_BF16, rows, cols, B.HQ_ROT_RIGHT, cfg, B.HQ_STAT_LSQ_GRAD,
        sc.data_ptr(), out.data_ptr(), ws.data_ptr(), nws, T.stream_ptr()), "lsq"), 2 * n2)
    res["qerr"] = timed(lambda: B.check(B.hq_rotated_stat(
        x.data_ptr(), None, B.HQ_BF16, rows, cols, B.HQ_ROT_RIGHT, cfg, B.HQ_STAT_QERR,
        sc.data_ptr(), out.data_ptr(), ws.data_ptr(), nws, T.stream_ptr()), "qerr"), n2)
    res["cold_start_step"] = timed(lambda: B.check(B.hq_cold_start_step(
        x.data_ptr(), B.HQ_BF16, rows, cols, B.HQ_ROT_RIGHT, cfg, step.data_ptr(), ws.data_ptr(),
        nws, T.stream_ptr()), "cold"), n2)
    cands = [16, 32, 64, 128, 256]
    carr = (ctypes.c_int32 * len(cands))(*cands)
    kb = ctypes.c_int32(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    B.check(B.hq_select_hadamard_k(x.data_ptr(), w.data_ptr(), B.HQ_BF16, rows, cols, D, cfg, carr,
                                   len(cands), kb, None, ws.data_ptr(), nws, T.stream_ptr()), "sel")
    res["select_k"] = {"candidates": cands, "chosen": kb.value,
                       "ms": round((time.perf_counter() - t0) * 1e3, 2),
                       "what": "absmax and error passes over X and W per candidate, synchronous"}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5,
                    help="workload id (default 5: HALO-2 step, 8192 x 13824 x 5120, k=128, the "
                         "largest layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=768)
    ap.add_argument("--check-configs", type=str, default="4,2",
                    help="also time these workloads' steps against three bf16 GEMMs (default "
                         "4,2: the Llama-7B-shaped MLP layer and the 2048 x 4096 x 4096 layer); "
                         "empty to skip")
    ap.add_argument("--no-qparams", action="store_true",
                    help="skip the quantizer-parameter statistics")
    ap.add_argument("--no-bmm", action="store_true",
                    help="skip the batched (attention) product")
    ap.add_argument("--no-lss", action="store_true",
                    help="skip the LSS-MM (sampled weight gradient) measurement")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 (E4M3) step of the same layer")
    ap.add_argument("--no-fp6", action="store_true",
                    help="skip the FP6 (E2M3, E3M2) steps of the same layer")
    ap.add_argument("--no-fwht", action="store_true",
                    help="skip the standalone hq_fwht bandwidth figure")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache prologue pass (kernel traces of the warm step)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB three times with a "
                         "plain device copy (reference dispatches for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
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

    ms_events = event_median_ms(step, warmup=2, reps=max(5, args.steps))

    # GEMM launches of each call of the step (one, or a head and a tail launch)
    per_call = []
    for name, call in (("fwd", lambda: layer.fwd(x, w, y, steps_t, stream)),
                       ("dx", (lambda: layer.bwd_input(dy, dx, steps_t, stream)) if dx is not None else None),
                       ("dw", (lambda: layer.bwd_weight(dw, stream)) if dw is not None else None)):
        if call is None:
            continue
        B.check(B.hq_profile_start(1 << B.HQ_KIND_GEMM), "profile")
        call()
        torch.cuda.synchronize()
        B.profile_stop_dict()
        per_call.append((name, len(B.profile_records())))

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
    recs = B.profile_records()
    ms_instr = (t3 - t2) * 1e3 / args.steps
    gcount, gms, gunits = prof["gemm"]
    gemm_tops = gunits / (gms * 1e-3) / 1e12 if gms > 0 else None
    gemm_avg_us = gms * 1e3 / gcount if gcount else None
    per_step = sum(n for _, n in per_call)
    products = {}
    if per_step and len(recs) == per_step * args.steps:
        pos = 0
        for name, n in per_call:
            for j in range(n):
                sel = [recs[st * per_step + pos + j] for st in range(args.steps)]
                ms_sum = sum(r[1] for r in sel)
                units = sum(r[2] for r in sel)
                label = name if n == 1 else "%s_%s" % (name, "head" if j == 0 else "tail")
                tops = units / (ms_sum * 1e-3) / 1e12
                products[label] = {"avg_us": round(ms_sum * 1e3 / len(sel), 2),
                                   "ops_per_launch": units / len(sel),
                                   "tops": round(tops, 1),
                                   "frac": round(tops / PEAK_INT8_TOPS, 4)}
            pos += n

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
        "ms_per_step_event_median": round(ms_events, 4),
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
            "products": products,
            "timing": "HIP events stamped by hipExtLaunchKernel on each GEMM launch, over a "
                      "second pass of the same %d steps (%.4f ms/step with the events); "
                      "achieved = all GEMM ops / all GEMM launch time" % (args.steps, ms_instr),
        },
        "breakdown_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in breakdown.items()},
    }
    if not args.no_bf16_baseline:
        try:
            ms_rb = bf16_baseline(cfg, "cublas")
            ms_lt = bf16_baseline(cfg, "cublaslt")
            result["bf16_baseline"] = {
                "what": "three unrotated bf16 torch.mm of the same shapes (Y, dX, dW), event "
                        "median of 20 after 5 warm-ups, against the HQ-MM step's event median",
                "ms_rocblas": round(ms_rb, 4), "ms_hipblaslt": round(ms_lt, 4),
                "speedup_vs_rocblas": round(ms_rb / ms_events, 3),
                "speedup_vs_hipblaslt": round(ms_lt / ms_events, 3)}
        except Exception as exc:  # report, do not fail the benchmark line
            result["bf16_baseline"] = {"error": str(exc)}
    checks = [int(c) for c in args.check_configs.split(",") if c.strip()]
    for cid in checks:
        if cid == args.config:
            continue
        print("[bench] step vs bf16 on config %d" % cid, file=sys.stderr, flush=True)
        try:
            result.setdefault("layer_vs_bf16", {})["config%d" % cid] = layer_vs_bf16(cid)
        except Exception as exc:  # report, do not fail the benchmark line
            result.setdefault("layer_vs_bf16", {})["config%d" % cid] = {"error": str(exc)}
    if not args.no_fp8 and cfg["bits"] == 8 and cfg["mode"] == WL.ABSMAX:
        print("[bench] fp8 step", file=sys.stderr, flush=True)
        try:
            result["fp8_step"] = fp8_step(args.config)
        except Exception as exc:  # report, do not fail the benchmark line
            result["fp8_step"] = {"error": str(exc)}
    if not args.no_fp6 and cfg["bits"] == 8 and cfg["mode"] == WL.ABSMAX:
        print("[bench] fp6 steps", file=sys.stderr, flush=True)
        for name, f in (("e2m3", WL.E2M3), ("e3m2", WL.E3M2)):
            try:
                result.setdefault("fp6_step", {})[name] = fp8_step(args.config, fmt=f)
            except Exception as exc:  # report, do not fail the benchmark line
                result.setdefault("fp6_step", {})[name] = {"error": str(exc)}
    if not args.no_qparams:
        print("[bench] quantizer-parameter statistics", file=sys.stderr, flush=True)
        try:
            result["qparams"] = qparam_stats()
        except Exception as exc:  # report, do not fail the benchmark line
            result["qparams"] = {"error": str(exc)}
    if not args.no_lss:
        print("[bench] LSS-MM weight gradient", file=sys.stderr, flush=True)
        for cid in (3, 4, 5):
            try:
                result.setdefault("lss_step", []).append(lss_step(cid))
            except Exception as exc:  # report, do not fail the benchmark line
                result.setdefault("lss_step", []).append({"config": cid, "error": str(exc)})
    if not args.no_bmm:
        print("[bench] batched attention product", file=sys.stderr, flush=True)
        try:
            result["bmm_step"] = bmm_step()
        except Exception as exc:  # report, do not fail the benchmark line
            result["bmm_step"] = {"error": str(exc)}
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
