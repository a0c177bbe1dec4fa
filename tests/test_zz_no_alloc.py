"""hq_linear_fwd_noalloc (the forward with its scratch in the library's fixed device array)
against hq_linear_fwd (the caller's workspace) on the same inputs: two calls in a row, the
second on a smaller layer, each must give the same codes, scales and output bit for bit (the
same kernels run on the same data). Called through the C ABI."""
import numpy as np
import pytest
import torch

from hadamard_rotated_precision_amd import binding as B
from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _fwd_both_ways(cfg):
    N, C, D, k = cfg["N"], cfg["C"], cfg["D"], cfg["k"]
    print("[case] no-alloc forward", N, C, D, k, flush=True)
    inputs = WL.make_inputs(cfg)
    x = T.device_tensor_from_bits(inputs["x"], cfg["in_dtype"])
    w = T.device_tensor_from_bits(inputs["w"], cfg["in_dtype"])
    out = []
    for noalloc in (False, True):
        layer = T.Layer(N, C, D, k, cfg["bits"], cfg["mode"], cfg["variant"])
        y = torch.full((N, D), 3.0, dtype=T.TORCH_DT[cfg["out_dtype"]], device="cuda")
        qxt = None if layer.qxt is None else layer.qxt.st
        args = (T.ptr(x), T.ptr(w), T.HQ_DT[x.dtype], N, C, D, layer.cfg, None, None, None,
                T.ptr(y), T.HQ_DT[y.dtype], layer.qx.st, qxt, layer.qw.st)
        if noalloc:
            B.check(B.hq_linear_fwd_noalloc(*args, T.stream_ptr()), "hq_linear_fwd_noalloc")
        else:
            B.check(B.hq_linear_fwd(*args, T.ptr(layer.ws), layer.ws_bytes, T.stream_ptr()),
                    "hq_linear_fwd")
        torch.cuda.synchronize()
        got = {"y": T.bits_of(y), "qx": layer.qx.codes_view().cpu().numpy(),
               "sx": float(layer.qx.scale.cpu()[0]), "qw": layer.qw.codes_view().cpu().numpy(),
               "qw_t": layer.qw.codes_t_view().cpu().numpy(), "sw": float(layer.qw.scale.cpu()[0])}
        if layer.qxt is not None:
            got["qxt"] = layer.qxt.codes_t_view().cpu().numpy()
            got["sxt"] = float(layer.qxt.scale.cpu()[0])
        out.append(got)
    ref, got = out
    assert ref.keys() == got.keys()
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)


def test_noalloc_forward_matches_workspace_forward_twice():
    # HALO-2, k = 128 with more 128 x 128 X items than workgroups (512 workgroups: the
    # two-sided partials fill the 1024 floats of a partials array)
    _fwd_both_ways(WL.config(5, N=2048, C=4352, D=256))
    # HALO-2, k = 256 (single-pass X over the grid barrier words in the scratch), then a
    # smaller layer whose X pass takes the two-launch path (absmax partials only)
    _fwd_both_ways(WL.config(2, N=512, C=1024, D=768))
    _fwd_both_ways(WL.config(2, N=256, C=512, D=256, k=64))
    # the HQ forward of the small fp16 layer, fp32 out
    _fwd_both_ways(WL.config(1, N=128, C=256, D=192))
