"""Shared helpers of the GPU parity tests: run the HIP path (through the C ABI) and the CPU
oracle on the same seeded inputs, and compare them.

Acceptance (for every workload):
  - integer GEMM outputs bit-exact given identical int8 codes;
  - codes within 1 LSB, on at most 1e-4 of the entries (fp32 rotation order vs the oracle's
    exact sums can move a value across a rounding boundary);
  - dequantized outputs with relative Frobenius error <= 1e-3 against the oracle's unrounded
    (double) value. An output stored in a 16-bit dtype also carries its own round-to-nearest,
    at most the unit roundoff u (2^-8 bf16, 2^-11 fp16) relative per element, so by the
    triangle inequality its bound is 1e-3 + u (1 + 1e-3); fp32 outputs get 1e-3 + 2^-24.
"""
import numpy as np
import torch

import oracle as O
from hadamard_rotated_precision_amd import binding as B
from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

CODE_FRAC = 1e-4
OUT_REL_FRO = 1e-3
UNIT_ROUNDOFF = {O.F32: 2.0 ** -24, O.F16: 2.0 ** -11, O.BF16: 2.0 ** -8}


def out_bound(dt):
    """Relative Frobenius bound of an output of dtype dt against the unrounded oracle."""
    u = UNIT_ROUNDOFF[dt]
    return OUT_REL_FRO + u * (1.0 + OUT_REL_FRO)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


_FP6_GRID = {}


def fp6_grid(fmt):
    """The non-negative values of an FP6 format, increasing (the oracle's grid, pinned against
    the hand-listed one in the FP6 pins)."""
    if fmt not in _FP6_GRID:
        top = O.fp6_max(fmt)
        sweep = np.linspace(0.0, top, 20001)
        _FP6_GRID[fmt] = np.unique(O.decode_e4m3(O.quantize_fp6(sweep, 1.0, fmt)))
    return _FP6_GRID[fmt]


def code_steps(codes, fmt=O.INT):
    """Codes as positions on their grid: the integer itself, for E4M3 bytes the signed
    magnitude code, for FP6 codes (kept as E4M3 bytes) the signed position on the FP6 grid
    (adjacent grid values are one apart; +0 and -0 are both 0)."""
    if fmt == O.E4M3:
        c = np.asarray(codes).view(np.uint8).astype(np.int16)
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    if fmt in (O.E2M3, O.E3M2):
        v = O.decode_e4m3(np.asarray(codes).view(np.uint8))
        grid = fp6_grid(fmt)
        pos = np.searchsorted(grid, np.abs(v))
        assert (grid[np.minimum(pos, grid.size - 1)] == np.abs(v)).all(), "a code off the FP6 grid"
        return np.where(v < 0, -pos, pos).astype(np.int16)
    return np.asarray(codes).astype(np.int16)


def code_diff(gpu, ref, fmt=O.INT):
    d = np.abs(code_steps(gpu, fmt) - code_steps(ref, fmt))
    return float((d != 0).mean()) if d.size else 0.0, int(d.max()) if d.size else 0


def assert_codes(gpu, ref, what, fmt=O.INT):
    frac, mx = code_diff(gpu, ref, fmt)
    print("[codes] %s mismatch fraction %.3g (max |diff| %d, %d entries)"
          % (what, frac, mx, gpu.size), flush=True)
    assert mx <= 1 and frac <= CODE_FRAC, "%s: mismatch frac %.3g max %d" % (what, frac, mx)
    return frac


def assert_out(gpu, exact, dt, what):
    """Output vs the oracle's unrounded value, within out_bound(dt); the error against the
    oracle rounded to the same dtype is printed beside it (context only)."""
    err = rel_fro(gpu, exact)
    matched = rel_fro(gpu, rounded(exact, dt)) if dt != O.F32 else err
    print("[out] %s rel fro %.3g vs exact (bound %.3g), %.3g vs dtype-rounded"
          % (what, err, out_bound(dt), matched), flush=True)
    assert err <= out_bound(dt), "%s: rel Frobenius %.3g > %.3g" % (what, err, out_bound(dt))
    return err


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


GUARD_BYTES = 4096      # canary band on each side of every output buffer
CANARY = 0xA5


def guarded_empty(shape, dtype, dev="cuda"):
    """An output tensor sitting between two canary bands (and itself pre-filled with the
    canary bytes). Returns (tensor, raw byte buffer); check_guards() verifies the bands."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    raw = torch.full((nbytes + 2 * GUARD_BYTES,), CANARY, dtype=torch.uint8, device=dev)
    t = raw[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)
    return t, raw


def check_guards(raws):
    """Every canary band still holds its bytes: no kernel wrote outside its output."""
    for name, raw in raws.items():
        head = raw[:GUARD_BYTES]
        tail = raw[raw.numel() - GUARD_BYTES:]
        assert bool((head == CANARY).all()), "%s: write before the output buffer" % name
        assert bool((tail == CANARY).all()), "%s: write past the output buffer" % name


def run_gpu(cfg, inputs, out_dt=None):
    """Run the configured passes through the C ABI; returns host copies of everything.
    Every output lies between canary bands, checked after the step."""
    dev = "cuda"
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    in_dt = cfg["in_dtype"]
    out_dt = cfg["out_dtype"] if out_dt is None else out_dt
    layer = T.Layer(N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"], device=dev,
                    fmt=cfg.get("fmt", O.INT))
    x = T.device_tensor_from_bits(inputs["x"], in_dt, dev)
    w = T.device_tensor_from_bits(inputs["w"], in_dt, dev)
    steps = None
    if cfg["mode"] == WL.STEP:
        steps = {n: torch.tensor([v], dtype=torch.float32, device=dev)
                 for n, v in inputs["steps"].items()}
    res = {"layer": layer}
    raws = {}
    y, raws["y"] = guarded_empty((N, D), T.TORCH_DT[out_dt], dev)
    layer.fwd(x, w, y, steps)
    res["y"] = y
    if "dx" in cfg["passes"] or "dw" in cfg["passes"]:
        dy = T.device_tensor_from_bits(inputs["dy"], in_dt, dev)
        dx, raws["dx"] = guarded_empty((N, C), T.TORCH_DT[out_dt], dev)
        layer.bwd_input(dy, dx, steps)
        res["dx"] = dx
        if "dw" in cfg["passes"]:
            dw, raws["dw"] = guarded_empty((D, C), T.TORCH_DT[out_dt], dev)
            layer.bwd_weight(dw)
            res["dw"] = dw
    torch.cuda.synchronize()
    check_guards(raws)
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
    return O.linear(X, W, dY, cfg["k"], cfg["bits"], cfg["variant"], cfg["mode"], steps, passes,
                    fmt=cfg.get("fmt", O.INT))


def compare_layer(cfg, h, ora, out_dt):
    """Full comparison of a (small) layer; returns a dict of measured figures."""
    stats = {}
    fmt = cfg.get("fmt", O.INT)
    stats["qx"] = assert_codes(h["qx"], ora["qx"], "qX", fmt)
    assert_scale(h["sx"], ora["sx"], "sX")
    stats["qw"] = assert_codes(h["qw"], ora["qw"], "qW", fmt)
    assert_scale(h["sw"], ora["sw"], "sW")
    np.testing.assert_array_equal(h["qw_t"], h["qw"].T)   # both layouts carry the same codes
    if "qx_t" in h:
        np.testing.assert_array_equal(h["qx_t"], h["qx"].T)
    if "qxt_t" in h:
        stats["qxt"] = assert_codes(h["qxt_t"].T, ora["qxt"], "qXt", fmt)
        assert_scale(h["sxt"], ora["sxt"], "sXt")
    if "qg" in h:
        stats["qg"] = assert_codes(h["qg"], ora["qg"], "qG", fmt)
        assert_scale(h["sg"], ora["sg"], "sG")
        np.testing.assert_array_equal(h["qg_t"], h["qg"].T)
    for name in ("y", "dx", "dw"):
        if name in h:
            stats[name] = assert_out(h[name], ora[name], out_dt, name)
    return stats


def outputs_from_gpu_codes(cfg, h):
    """The oracle's products evaluated on the GPU's own codes and scales (isolates the
    GEMM + epilogue from code flips)."""
    k, v, f = cfg["k"], cfg["variant"], cfg.get("fmt", O.INT)
    cv = (lambda q: np.asarray(q).view(np.uint8)) if f in O.FLOAT_FORMATS else (lambda q: q)
    out = {"y": O.fwd_from_codes(cv(h["qx"]), h["sx"], cv(h["qw"]), h["sw"], k, v, fmt=f)}
    if "qg" in h:
        if "dx" in h:
            out["dx"] = O.bwd_input_from_codes(cv(h["qg"]), h["sg"], cv(h["qw"]), h["sw"], k, v,
                                               fmt=f)
        if "dw" in h:
            if v == O.HALO2:
                out["dw"] = O.bwd_weight_from_codes(cv(h["qg"]), h["sg"], cv(h["qxt_t"].T),
                                                    h["sxt"], k, v, fmt=f)
            else:
                out["dw"] = O.bwd_weight_from_codes(cv(h["qg"]), h["sg"], cv(h["qx"]), h["sx"],
                                                    k, v, fmt=f)
    return out


def fullsize_sampled(cfg, seed, dw_rows=()):
    """A workload's whole step at its full size: codes and scales compared in full against the
    oracle's, outputs on sampled rows / k-aligned blocks against the oracle's exact values on
    its own codes (plus 64-row dW blocks at dw_rows). The format and the code width come from
    cfg."""
    N, C, D, k, v = cfg["N"], cfg["C"], cfg["D"], cfg["k"], cfg["variant"]
    bits, f = cfg["bits"], cfg.get("fmt", O.INT)
    out_dt = cfg["out_dtype"]
    inputs = WL.make_inputs(cfg)
    res = run_gpu(cfg, inputs)
    L = res["layer"]
    X = O.decode(inputs["x"], cfg["in_dtype"])
    qx, sx, qxt, sxt = O.quantize_x(X, k, bits, v, fmt=f)
    del X
    assert_codes(L.qx.codes_view().cpu().numpy(), qx, "qX", f)
    assert_scale(float(L.qx.scale.cpu()[0]), sx, "sX")
    assert_codes(L.qxt.codes_t_view().cpu().numpy().T, qxt, "qXt", f)
    assert_scale(float(L.qxt.scale.cpu()[0]), sxt, "sXt")
    W = O.decode(inputs["w"], cfg["in_dtype"])
    qw, sw = O.quantize_w(W, k, bits, v, fmt=f)
    del W
    assert_codes(L.qw.codes_view().cpu().numpy(), qw, "qW", f)
    G = O.decode(inputs["dy"], cfg["in_dtype"])
    qg, sg = O.quantize_g(G, k, bits, v, fmt=f)
    del G
    assert_codes(L.qg.codes_view().cpu().numpy(), qg, "qG", f)
    rng = np.random.default_rng(seed)
    rs = np.sort(rng.choice(N, 128, replace=False))
    cs = np.sort(rng.choice(D, 128, replace=False))
    y = O.decode(T.bits_of(res["y"][rs][:, cs].contiguous()), out_dt)
    assert_out(y, O.fwd_from_codes(qx, sx, qw, sw, k, v, rows=rs, cols=cs, fmt=f), out_dt, "Y")
    for _ in range(2):
        r0, c0 = int(rng.integers(0, N // k)) * k, int(rng.integers(0, C // k)) * k
        ref = O.bwd_input_from_codes(qg, sg, qw, sw, k, v, row_block=(r0, k), col_block=(c0, k),
                                     fmt=f)
        got = O.decode(T.bits_of(res["dx"][r0:r0 + k, c0:c0 + k].contiguous()), out_dt)
        assert_out(got, ref, out_dt, "dX block (%d, %d)" % (r0, c0))
        r0, c0 = int(rng.integers(0, D - 64 + 1)), int(rng.integers(0, C // k)) * k
        ref = O.bwd_weight_from_codes(qg, sg, qxt, sxt, k, v, row_block=(r0, 64),
                                      col_block=(c0, k), fmt=f)
        got = O.decode(T.bits_of(res["dw"][r0:r0 + 64, c0:c0 + k].contiguous()), out_dt)
        assert_out(got, ref, out_dt, "dW block (%d, %d)" % (r0, c0))
    for r0 in dw_rows:
        c0 = int(rng.integers(0, C // k)) * k
        ref = O.bwd_weight_from_codes(qg, sg, qxt, sxt, k, v, row_block=(r0, 64),
                                      col_block=(c0, k), fmt=f)
        got = O.decode(T.bits_of(res["dw"][r0:r0 + 64, c0:c0 + k].contiguous()), out_dt)
        assert_out(got, ref, out_dt, "dW block (%d, %d)" % (r0, c0))
