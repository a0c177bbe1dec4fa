"""Two layer steps on two streams at once, each with its own workspace and outputs.

The calls keep no state between launches, and every wait inside a launch is bounded: the grid
barrier of the single-pass X kernel gives up and leaves the work to the fixup launch when not
every workgroup is resident, and a tile of a dX pair stops waiting for its partner and finishes
alone. So two steps sharing the GPU must give exactly what each gives alone, whichever way their
workgroups interleave.
"""
import pytest
import torch

from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"


class _Step:
    def __init__(self, cfg, seed):
        cfg = dict(cfg, seed=seed)
        self.N, self.C, self.D = cfg["N"], cfg["C"], cfg["D"]
        inputs = WL.make_inputs(cfg)
        self.x = T.device_tensor_from_bits(inputs["x"], cfg["in_dtype"], DEV)
        self.w = T.device_tensor_from_bits(inputs["w"], cfg["in_dtype"], DEV)
        self.dy = T.device_tensor_from_bits(inputs["dy"], cfg["in_dtype"], DEV)
        self.layer = T.Layer(self.N, self.C, self.D, cfg["k"], cfg["bits"], cfg["mode"],
                             cfg["variant"], device=DEV)
        odt = T.TORCH_DT[cfg["out_dtype"]]
        self.y = torch.empty((self.N, self.D), dtype=odt, device=DEV)
        self.dx = torch.empty((self.N, self.C), dtype=odt, device=DEV)
        self.dw = torch.empty((self.D, self.C), dtype=odt, device=DEV)

    def run(self, stream):
        self.layer.fwd(self.x, self.w, self.y, None, stream)
        self.layer.bwd_input(self.dy, self.dx, None, stream)
        self.layer.bwd_weight(self.dw, stream)

    def outputs(self):
        return [t.clone() for t in (self.y, self.dx, self.dw)]


@pytest.mark.parametrize("shape", [dict(N=512, C=768, D=512), dict(N=2048, C=4096, D=4096)])
def test_two_streams_match_alone(shape):
    cfg = WL.config(2, **shape)
    print("[case] streams", shape, flush=True)
    a, b = _Step(cfg, 201), _Step(cfg, 202)
    main = torch.cuda.current_stream()
    a.run(main)
    b.run(main)
    torch.cuda.synchronize()
    ref_a, ref_b = a.outputs(), b.outputs()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for t in (a.y, a.dx, a.dw, b.y, b.dx, b.dw):
            t.fill_(0)
        torch.cuda.synchronize()
        a.run(s1)
        b.run(s2)
        torch.cuda.synchronize()
        for name, got, ref in zip(("y", "dx", "dw"), a.outputs(), ref_a):
            assert torch.equal(got, ref), ("a", rep, name)
        for name, got, ref in zip(("y", "dx", "dw"), b.outputs(), ref_b):
            assert torch.equal(got, ref), ("b", rep, name)
