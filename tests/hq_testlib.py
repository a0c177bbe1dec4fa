"""Shared helpers of the GPU parity tests: run the HIP path (through the C ABI) and the CPU
oracle on the same seeded inputs, and compare them.

Acceptance (for every workload):
  - integer GEMM outputs bit-exact given identical int8 codes;
  - codes within 1 LSB, on at most 1e-4 of the entries (fp32 rotation order vs the oracle's
    exact sums can move a value across a rounding boundary);
  - dequantized outputs with relative Frobenius error <= 1e-3 against the oracle rounded to
    the same output dtype.
"""
import numpy as np
import torch

import oracle as O
from hadamard_rotated_precision_amd import binding as B
from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

CODE_FRAC = 1e-4
OUT_REL_FRO = 1e-3


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def code_diff(gpu, ref):
    d = np.abs(gpu.astype(np.int16) - ref.astype(np.int16))
    return float((d != 0).mean()) if d.size else 0.0, int(d.max()) if d.size else 0


def assert_codes(gpu, ref, what):
    frac, mx = code_diff(gpu, ref)
    assert mx <= 1 and frac <= CODE_FRAC, "%s: mismatch frac %.3g max %d" % (what, frac, mx)
    return frac


def assert_scale(gpu, ref, what):
    g, r = np.float32(gpu), np.float32(ref)
    if r == 0:
        assert g == 0, what
        return
    # the GPU max is over fp32 values rotated in a different order: allow a few ulp
    assert abs(float(g) - float(r)) <= 4 * np.spacing(r), "%s: %r vs %r" % (what, g, r)


def decode_out(bits, dt):
    return O.decode(bits, dt)


def rounded(vals, dt):
    """Oracle doubles rounded to the output dtype and decoded back to doubles."""
    return O.decode(O.round_to(vals, dt), dt)


def run_gpu(cfg, inputs, out_dt=None):
    """Run the configured passes through the C ABI; returns host copies of everything."""
    dev = "cuda"
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    in_dt = cfg["in_dtype"]
    out_dt = cfg["out_dtype"] if out_dt is None else out_dt
    layer = T.Layer(N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"], device=dev)
    x = T.device_tensor_from_bits(inputs["x"], in_dt, dev)
    w = T.device_tensor_from_bits(inputs["w"], in_dt, dev)
    steps = None
    if cfg["mode"] == WL.STEP:
        steps = {n: torch.tensor([v], dtype=torch.float32, device=dev)
                 for n, v in inputs["steps"].items()}
    res = {"layer": layer}
    y = torch.empty((N, D), dtype=T.TORCH_DT[out_dt], device=dev)
    layer.fwd(x, w, y, steps)
    res["y"] = y
    if "dx" in cfg["passes"] or "dw" in cfg["passes"]:
        dy = T.device_tensor_from_bits(inputs["dy"], in_dt, dev)
        dx = torch.empty((N, C), dtype=T.TORCH_DT[out_dt], device=dev)
        layer.bwd_input(dy, dx, steps)
        res["dx"] = dx
        if "dw" in cfg["passes"]:
            dw = torch.empty((D, C), dtype=T.TORCH_DT[out_dt], device=dev)
            layer.bwd_weight(dw)
            res["dw"] = dw
    torch.cuda.synchronize()
    return res


def host(res, out_dt):
    """Copy GPU results to host numpy: codes (without pitch padding), scales, outputs."""
    L = res["layer"]
    h = {}
    h["qx"] = L.qx.codes_view().cpu().numpy()
    h["sx"] = float(L.qx.scale.cpu()[0])
    if L.qx.codes_t is not None:
        h["qx_t"] = L.qx.codes_t_view().cpu().numpy()
    if L.qxt is not None:
        h["qxt_t"] = L.qxt.codes_t_view().cpu().numpy()
        h["sxt"] = float(L.qxt.scale.cpu()[0])
    h["qw"] = L.qw.codes_view().cpu().numpy()
    h["qw_t"] = L.qw.codes_t_view().cpu().numpy()
    h["sw"] = float(L.qw.scale.cpu()[0])
    for name in ("y", "dx", "dw"):
        if name in res:
            h[name] = decode_out(T.bits_of(res[name]), out_dt)
    if "dx" in res:
        h["qg"] = L.qg.codes_view().cpu().numpy()
        h["qg_t"] = L.qg.codes_t_view().cpu().numpy()
        h["sg"] = float(L.qg.scale.cpu()[0])
    return h


def run_oracle(cfg, inputs):
    in_dt = cfg["in_dtype"]
    X = O.decode(inputs["x"], in_dt)
    W = O.decode(inputs["w"], in_dt)
    dY = O.decode(inputs["dy"], in_dt) if inputs.get("dy") is not None else None
    steps = inputs.get("steps")
    passes = cfg["passes"]
    return O.linear(X, W, dY, cfg["k"], cfg["bits"], cfg["variant"], cfg["mode"], steps, passes)


def compare_layer(cfg, h, ora, out_dt):
    """Full comparison of a (small) layer; returns a dict of measured figures."""
    stats = {}
    stats["qx"] = assert_codes(h["qx"], ora["qx"], "qX")
    assert_scale(h["sx"], ora["sx"], "sX")
    stats["qw"] = assert_codes(h["qw"], ora["qw"], "qW")
    assert_scale(h["sw"], ora["sw"], "sW")
    np.testing.assert_array_equal(h["qw_t"], h["qw"].T)   # both layouts carry the same codes
    if "qx_t" in h:
        np.testing.assert_array_equal(h["qx_t"], h["qx"].T)
    if "qxt_t" in h:
        stats["qxt"] = assert_codes(h["qxt_t"].T, ora["qxt"], "qXt")
        assert_scale(h["sxt"], ora["sxt"], "sXt")
    if "qg" in h:
        stats["qg"] = assert_codes(h["qg"], ora["qg"], "qG")
        assert_scale(h["sg"], ora["sg"], "sG")
        np.testing.assert_array_equal(h["qg_t"], h["qg"].T)
    for name in ("y", "dx", "dw"):
        if name in h:
            err = rel_fro(h[name], rounded(ora[name], out_dt))
            stats[name] = err
            assert err <= OUT_REL_FRO, "%s: rel Frobenius %.3g" % (name, err)
    return stats


def outputs_from_gpu_codes(cfg, h):
    """The oracle's products evaluated on the GPU's own codes and scales (isolates the
    GEMM + epilogue from code flips)."""
    k, v = cfg["k"], cfg["variant"]
    out = {"y": O.fwd_from_codes(h["qx"], h["sx"], h["qw"], h["sw"], k, v)}
    if "qg" in h:
        if "dx" in h:
            out["dx"] = O.bwd_input_from_codes(h["qg"], h["sg"], h["qw"], h["sw"], k, v)
        if "dw" in h:
            if v == O.HALO2:
                out["dw"] = O.bwd_weight_from_codes(h["qg"], h["sg"], h["qxt_t"].T, h["sxt"], k, v)
            else:
                out["dw"] = O.bwd_weight_from_codes(h["qg"], h["sg"], h["qx"], h["sx"], k, v)
    return out
