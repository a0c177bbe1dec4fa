"""GPU parity of the batched HQ-MM (attention BMMs, INT4 page §A.1) against the oracle,
through hq_bmm_fwd / hq_bmm_bwd_input / hq_bmm_bwd_weight: codes and the one scale of each
batched tensor, and every batch's outputs, against oracle.linear_batched on the same inputs.
Bars as for the layer (hq_testlib): codes within 1 step on <= 1e-4, outputs within
out_bound of the unrounded oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from hadamard_rotated_precision_amd import binding as B
from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

from hq_testlib import (assert_codes, assert_out, assert_scale, check_guards, guarded_empty,
                        rel_fro)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_bmm(cfg, inputs, out_dt):
    nb, N, C, D = cfg["batch"], cfg["N"], cfg["C"], cfg["D"]
    in_dt = cfg["in_dtype"]
    L = T.BatchedLayer(nb, N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"],
                       fmt=cfg.get("fmt", O.INT))
    x = T.device_tensor_from_bits(inputs["x"], in_dt)
    w = T.device_tensor_from_bits(inputs["w"], in_dt)
    dy = T.device_tensor_from_bits(inputs["dy"], in_dt)
    odt = T.TORCH_DT[out_dt]
    raws = {}
    y, raws["y"] = guarded_empty((nb, N, D), odt)
    dx, raws["dx"] = guarded_empty((nb, N, C), odt)
    dw, raws["dw"] = guarded_empty((nb, D, C), odt)
    L.fwd(x, w, y)
    L.bwd_input(dy, dx)
    L.bwd_weight(dw)
    torch.cuda.synchronize()
    check_guards(raws)
    return L, {"y": y, "dx": dx, "dw": dw}


def check(cfg, out_dt):
    inputs = WL.make_batched_inputs(cfg)
    L, outs = run_bmm(cfg, inputs, out_dt)
    f = cfg.get("fmt", O.INT)
    dt = cfg["in_dtype"]
    ref = O.linear_batched(O.decode(inputs["x"], dt), O.decode(inputs["w"], dt),
                           O.decode(inputs["dy"], dt), cfg["k"], cfg["bits"], cfg["variant"],
                           fmt=f)
    assert_codes(L.qx.codes_view().cpu().numpy(), ref["qx"], "qX", f)
    assert_scale(float(L.qx.scale.cpu()[0]), ref["sx"], "sX")
    assert_codes(L.qw.codes_view().cpu().numpy(), ref["qw"], "qW", f)
    assert_scale(float(L.qw.scale.cpu()[0]), ref["sw"], "sW")
    assert_codes(L.qg.codes_view().cpu().numpy(), ref["qg"], "qG", f)
    assert_scale(float(L.qg.scale.cpu()[0]), ref["sg"], "sG")
    if L.qxt is not None:
        assert_codes(L.qxt.codes_t_view().cpu().numpy().T, ref["qxt"], "qXt", f)
        assert_scale(float(L.qxt.scale.cpu()[0]), ref["sxt"], "sXt")
    for name in ("y", "dx", "dw"):
        got = O.decode(T.bits_of(outs[name]), out_dt)
        assert_out(got, ref[name], out_dt, name)
        # every batch on its own (a batch offset mistake shows here even if the total passes)
        for b in range(cfg["batch"]):
            assert rel_fro(got[b], ref[name][b]) <= 4 * (1e-3 + 2.0 ** -8), (name, b)


@pytest.mark.parametrize("variant", [B.HQ_VARIANT_HALO2, B.HQ_VARIANT_HQ, B.HQ_VARIANT_HALO0])
@pytest.mark.parametrize("out_dt", [O.BF16, O.F32])
def test_bmm_attention_shapes(variant, out_dt):
    cfg = WL.attention_config(batch=6, N=256, D=192, k=64, variant=variant)
    print("[case] bmm", variant, out_dt, flush=True)
    check(cfg, out_dt)


@pytest.mark.parametrize("batch,N,C,D,k", [(3, 64, 128, 80, 16), (2, 32, 256, 48, 32),
                                           (1, 256, 128, 256, 128), (40, 128, 64, 128, 64)])
def test_bmm_ragged_and_many_batches(batch, N, C, D, k):
    """Tiles that end inside a batch (D = 80, 48), one batch (the layer path), and enough
    batches for the grid to fill the device with 128-wide tiles."""
    cfg = WL.attention_config(batch=batch, N=N, C=C, D=D, k=k)
    print("[case] bmm", batch, N, C, D, k, flush=True)
    check(cfg, O.F32)


def test_bmm_fp8():
    cfg = WL.attention_config(batch=4, N=256, D=256, k=128, fmt=WL.E4M3)
    print("[case] bmm fp8", flush=True)
    check(cfg, O.F32)


def test_bmm_equals_layers_with_shared_steps():
    """With one given step per tensor (STEP mode) the batched calls and one layer call per
    batch run the same kernels on the same codes: outputs equal bit for bit."""
    cfg = WL.attention_config(batch=3, N=128, D=128, k=64)
    nb, N, C, D, k = cfg["batch"], cfg["N"], cfg["C"], cfg["D"], cfg["k"]
    inputs = WL.make_batched_inputs(cfg)
    dt = cfg["in_dtype"]
    steps = {n: torch.tensor([v], dtype=torch.float32, device=DEV)
             for n, v in {"x": 0.2, "xt": 3.0, "w": 0.2, "g": 3e-5}.items()}
    x = T.device_tensor_from_bits(inputs["x"], dt)
    w = T.device_tensor_from_bits(inputs["w"], dt)
    dy = T.device_tensor_from_bits(inputs["dy"], dt)
    L = T.BatchedLayer(nb, N, C, D, k, 8, B.HQ_SCALE_STEP, B.HQ_VARIANT_HALO2)
    yb = torch.empty((nb, N, D), dtype=torch.float32, device=DEV)
    dxb = torch.empty((nb, N, C), dtype=torch.float32, device=DEV)
    dwb = torch.empty((nb, D, C), dtype=torch.float32, device=DEV)
    L.fwd(x, w, yb, steps)
    L.bwd_input(dy, dxb, steps)
    L.bwd_weight(dwb)
    for b in range(nb):
        l1 = T.Layer(N, C, D, k, 8, B.HQ_SCALE_STEP, B.HQ_VARIANT_HALO2)
        y = torch.empty((N, D), dtype=torch.float32, device=DEV)
        dx = torch.empty((N, C), dtype=torch.float32, device=DEV)
        dw = torch.empty((D, C), dtype=torch.float32, device=DEV)
        l1.fwd(x[b].contiguous(), w[b].contiguous(), y, steps)
        l1.bwd_input(dy[b].contiguous(), dx, steps)
        l1.bwd_weight(dw)
        torch.cuda.synchronize()
        assert torch.equal(y, yb[b]) and torch.equal(dx, dxb[b]) and torch.equal(dw, dwb[b]), b


@pytest.mark.timeout(900)
def test_bmm_fullsize_attention_sampled():
    """The attention-score products at the size bench.py times them (128 batches = 4 sequences
    x 32 heads, 1024 tokens, head width 128, k = 128, HALO-2): the stacked codes and the shared
    scales in full, the products of three batches (first, middle, last) against the oracle's
    exact values on its own codes."""
    cfg = WL.attention_config()
    nb, N, C, D, k, v = cfg["batch"], cfg["N"], cfg["C"], cfg["D"], cfg["k"], cfg["variant"]
    print("[case] bmm fullsize", cfg["name"], flush=True)
    inputs = WL.make_batched_inputs(cfg)
    L, outs = run_bmm(cfg, inputs, cfg["out_dtype"])
    dt, out_dt = cfg["in_dtype"], cfg["out_dtype"]
    qx, sx, qxt, sxt = O.quantize_x(O.decode(inputs["x"], dt).reshape(nb * N, C), k, cfg["bits"], v)
    qw, sw = O.quantize_w(O.decode(inputs["w"], dt).reshape(nb * D, C), k, cfg["bits"], v)
    qg, sg = O.quantize_g(O.decode(inputs["dy"], dt).reshape(nb * N, D), k, cfg["bits"], v)
    assert_codes(L.qx.codes_view().cpu().numpy(), qx, "qX")
    assert_scale(float(L.qx.scale.cpu()[0]), sx, "sX")
    assert_codes(L.qw.codes_view().cpu().numpy(), qw, "qW")
    assert_scale(float(L.qw.scale.cpu()[0]), sw, "sW")
    assert_codes(L.qg.codes_view().cpu().numpy(), qg, "qG")
    assert_scale(float(L.qg.scale.cpu()[0]), sg, "sG")
    assert_codes(L.qxt.codes_t_view().cpu().numpy().T, qxt, "qXt")
    assert_scale(float(L.qxt.scale.cpu()[0]), sxt, "sXt")
    print("[step] codes compared", flush=True)
    for b in (0, nb // 2 - 7, nb - 1):
        xs, ws = slice(b * N, (b + 1) * N), slice(b * D, (b + 1) * D)
        refs = {"y": O.fwd_from_codes(qx[xs], sx, qw[ws], sw, k, v),
                "dx": O.bwd_input_from_codes(qg[xs], sg, qw[ws], sw, k, v),
                "dw": O.bwd_weight_from_codes(qg[xs], sg, qxt[xs], sxt, k, v)}
        for name, ref in refs.items():
            got = O.decode(T.bits_of(outs[name][b].contiguous()), out_dt)
            assert_out(got, ref, out_dt, "%s batch %d" % (name, b))
