"""The three calls of a layer step inside one captured HIP graph.

Every launch of the library is a kernel (the barrier words, tile-pair flags and STEP-mode
scales are cleared or written by small kernels, never by a memset), no call synchronizes with
the host or allocates, so a caller can capture a whole step and replay it. Each replay must
give the eager step's results bit for bit: outputs, codes and scales, with the codes and
outputs overwritten with junk before every replay and eager steps (and host synchronizations)
run between the replays.
"""
import pytest
import torch

from hadamard_rotated_precision_amd import tensors as T
from hadamard_rotated_precision_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"

# small shapes of three workloads: HALO-2 with the single-pass X prologue and the tile-pair
# dX epilogue (k = 256), HQ with INT4-range STEP scales (fwd + dX), HALO-2 at k = 128
CASES = [
    (2, dict(N=512, C=768, D=512)),
    (3, dict(N=1000, C=1024, D=1000)),
    (5, dict(N=256, C=1408, D=640)),
]


def _state(layer, outs):
    """Everything a step writes: outputs, then codes and scales of each saved tensor."""
    got = [o.clone() for o in outs]
    for q in (layer.qx, layer.qxt, layer.qw, layer.qg):
        if q is None:
            continue
        for buf in (q.codes_view(), q.codes_t_view(), q.scale):
            if buf is not None:
                got.append(buf.clone())
    return got


def _scramble(layer, outs):
    for o in outs:
        o.fill_(3.0)
    for q in (layer.qx, layer.qxt, layer.qw, layer.qg):
        if q is None:
            continue
        for buf in (q.codes, q.codes_t):
            if buf is not None:
                buf.fill_(85)
        q.scale.fill_(-1.0)


@pytest.mark.parametrize("cid,shape", CASES)
def test_step_graph_replay_matches_eager(cid, shape):
    cfg = WL.config(cid, **shape)
    print("[case] graph", cfg["name"], cfg["N"], cfg["C"], cfg["D"], flush=True)
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    inputs = WL.make_inputs(cfg)
    x = T.device_tensor_from_bits(inputs["x"], cfg["in_dtype"], DEV)
    w = T.device_tensor_from_bits(inputs["w"], cfg["in_dtype"], DEV)
    dy = T.device_tensor_from_bits(inputs["dy"], cfg["in_dtype"], DEV)
    steps = None
    if cfg["mode"] == WL.STEP:
        steps = {n: torch.tensor([v], dtype=torch.float32, device=DEV)
                 for n, v in inputs["steps"].items()}
    layer = T.Layer(N, C, D, cfg["k"], cfg["bits"], cfg["mode"], cfg["variant"], device=DEV)
    odt = T.TORCH_DT[cfg["out_dtype"]]
    outs = [torch.empty((N, D), dtype=odt, device=DEV), torch.empty((N, C), dtype=odt, device=DEV)]
    with_dw = "dw" in cfg["passes"]
    if with_dw:
        outs.append(torch.empty((D, C), dtype=odt, device=DEV))

    def step(stream):
        layer.fwd(x, w, outs[0], steps, stream)
        layer.bwd_input(dy, outs[1], steps, stream)
        if with_dw:
            layer.bwd_weight(outs[2], stream)

    # the reference is an eager step over the same junk, so that buffers a variant leaves
    # unwritten compare equal too
    main = torch.cuda.current_stream()
    _scramble(layer, outs)
    step(main)
    torch.cuda.synchronize()
    ref = _state(layer, outs)

    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        step(side)
    main.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(3):
        _scramble(layer, outs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _state(layer, outs)
        assert len(got) == len(ref)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (cfg["name"], rep, i)
        step(main)   # eager work between replays
        torch.cuda.synchronize()
    del graph
