"""Device-memory plumbing around the C ABI: torch allocates the buffers (codes, scales,
outputs, workspace) and names the stream; the binding passes raw pointers to libhq.
No arithmetic of the method happens here."""
import numpy as np
import torch

from . import binding as B

TORCH_DT = {B.HQ_F32: torch.float32, B.HQ_F16: torch.float16, B.HQ_BF16: torch.bfloat16}
HQ_DT = {torch.float32: B.HQ_F32, torch.float16: B.HQ_F16, torch.bfloat16: B.HQ_BF16}


def pitch16(n):
    return (n + 15) // 16 * 16


def ptr(t):
    return None if t is None else t.data_ptr()


def stream_ptr(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def device_tensor_from_bits(bits, dtype, device="cuda"):
    """Upload a host array of raw bits (uint16 for fp16/bf16, float32 for fp32)."""
    if dtype == B.HQ_F32:
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def bits_of(t):
    """Raw host bits of a device tensor (uint16 for 16-bit dtypes, float32 for fp32)."""
    h = t.detach().cpu()
    if h.dtype == torch.float32:
        return h.numpy()
    return h.view(torch.int16).numpy().view(np.uint16)


class QTensor:
    """Caller-owned storage of one quantized tensor: codes (rows x pitch), codes_t
    (cols x pitch), one device float scale, and the hq_qtensor struct pointing at them."""

    def __init__(self, rows, cols, codes=True, codes_t=True, device="cuda"):
        self.rows, self.cols = rows, cols
        self.codes = (torch.empty((rows, pitch16(cols)), dtype=torch.int8, device=device)
                      if codes else None)
        self.codes_t = (torch.empty((cols, pitch16(rows)), dtype=torch.int8, device=device)
                        if codes_t else None)
        self.scale = torch.zeros(1, dtype=torch.float32, device=device)
        self.st = B.hq_qtensor()
        self.st.codes = ptr(self.codes)
        self.st.codes_t = ptr(self.codes_t)
        self.st.scale = ptr(self.scale)
        self.st.ld = pitch16(cols)
        self.st.ld_t = pitch16(rows)

    def codes_view(self):
        return None if self.codes is None else self.codes[:, :self.cols]

    def codes_t_view(self):
        return None if self.codes_t is None else self.codes_t[:, :self.rows]


def config(k, bits, scale_mode, variant, fmt=B.HQ_FMT_INT):
    c = B.hq_config()
    c.k, c.bits, c.scale_mode, c.variant, c.format = k, bits, scale_mode, variant, fmt
    return c


class Layer:
    """Buffers for one linear layer (N tokens, C in, D out) and the three HQ-MM calls."""

    def __init__(self, N, C, D, k, bits, scale_mode, variant, device="cuda", fmt=B.HQ_FMT_INT):
        self.N, self.C, self.D = N, C, D
        self.cfg = config(k, bits, scale_mode, variant, fmt)
        self.variant = variant
        self.ws_bytes = B.hq_workspace_bytes(self.cfg, N, C, D)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)
        halo2 = variant == B.HQ_VARIANT_HALO2
        self.qx = QTensor(N, C, codes=True, codes_t=not halo2, device=device)
        self.qxt = QTensor(N, C, codes=False, codes_t=True, device=device) if halo2 else None
        self.qw = QTensor(D, C, codes=True, codes_t=True, device=device)
        self.qg = QTensor(N, D, codes=True, codes_t=True, device=device)

    def fwd(self, x, w, y, steps=None, stream=None):
        steps = steps or {}
        B.check(B.hq_linear_fwd(
            ptr(x), ptr(w), HQ_DT[x.dtype], self.N, self.C, self.D, self.cfg,
            ptr(steps.get("x")), ptr(steps.get("w")), ptr(steps.get("xt", steps.get("x"))),
            ptr(y), HQ_DT[y.dtype], self.qx.st, None if self.qxt is None else self.qxt.st,
            self.qw.st, ptr(self.ws), self.ws_bytes, stream_ptr(stream)), "hq_linear_fwd")

    def bwd_input(self, dy, dx, steps=None, stream=None):
        steps = steps or {}
        B.check(B.hq_linear_bwd_input(
            ptr(dy), HQ_DT[dy.dtype], self.N, self.C, self.D, self.cfg, ptr(steps.get("g")),
            self.qw.st, ptr(dx), HQ_DT[dx.dtype], self.qg.st, ptr(self.ws), self.ws_bytes,
            stream_ptr(stream)), "hq_linear_bwd_input")

    def bwd_weight(self, dw, stream=None):
        qx = self.qxt if self.qxt is not None else self.qx
        B.check(B.hq_linear_bwd_weight(
            self.qg.st, qx.st, self.N, self.C, self.D, self.cfg, ptr(dw), HQ_DT[dw.dtype],
            ptr(self.ws), self.ws_bytes, stream_ptr(stream)), "hq_linear_bwd_weight")


class BatchedLayer:
    """Buffers for a batched product (batch x (N x C) by batch x (D x C), e.g. attention
    heads) and the three batched calls; codes describe the stacked matrices."""

    def __init__(self, batch, N, C, D, k, bits, scale_mode, variant, device="cuda",
                 fmt=B.HQ_FMT_INT):
        self.batch, self.N, self.C, self.D = batch, N, C, D
        self.cfg = config(k, bits, scale_mode, variant, fmt)
        self.variant = variant
        self.ws_bytes = B.hq_bmm_workspace_bytes(self.cfg)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)
        halo2 = variant == B.HQ_VARIANT_HALO2
        NB, DB = batch * N, batch * D
        self.qx = QTensor(NB, C, codes=True, codes_t=not halo2, device=device)
        self.qxt = QTensor(NB, C, codes=False, codes_t=True, device=device) if halo2 else None
        self.qw = QTensor(DB, C, codes=True, codes_t=True, device=device)
        self.qg = QTensor(NB, D, codes=True, codes_t=True, device=device)

    def fwd(self, x, w, y, steps=None, stream=None):
        steps = steps or {}
        B.check(B.hq_bmm_fwd(
            ptr(x), ptr(w), HQ_DT[x.dtype], self.batch, self.N, self.C, self.D, self.cfg,
            ptr(steps.get("x")), ptr(steps.get("w")), ptr(steps.get("xt", steps.get("x"))),
            ptr(y), HQ_DT[y.dtype], self.qx.st, None if self.qxt is None else self.qxt.st,
            self.qw.st, ptr(self.ws), self.ws_bytes, stream_ptr(stream)), "hq_bmm_fwd")

    def bwd_input(self, dy, dx, steps=None, stream=None):
        steps = steps or {}
        B.check(B.hq_bmm_bwd_input(
            ptr(dy), HQ_DT[dy.dtype], self.batch, self.N, self.C, self.D, self.cfg,
            ptr(steps.get("g")), self.qw.st, ptr(dx), HQ_DT[dx.dtype], self.qg.st, ptr(self.ws),
            self.ws_bytes, stream_ptr(stream)), "hq_bmm_bwd_input")

    def bwd_weight(self, dw, stream=None):
        qx = self.qxt if self.qxt is not None else self.qx
        B.check(B.hq_bmm_bwd_weight(
            self.qg.st, qx.st, self.batch, self.N, self.C, self.D, self.cfg, ptr(dw),
            HQ_DT[dw.dtype], ptr(self.ws), self.ws_bytes, stream_ptr(stream)), "hq_bmm_bwd_weight")


class LssGrad:
    """Buffers for the sampled weight gradient (hq_lss_bwd_weight) of an N x C -> D layer:
    workspace, probabilities, kept-token list and the stats record (kept, s8, s_hi, s_lo)."""

    def __init__(self, N, C, D, k, variant=B.HQ_VARIANT_HQ, device="cuda"):
        self.N, self.C, self.D = N, C, D
        self.cfg = config(k, 4, B.HQ_SCALE_ABSMAX, variant)
        self.ws_bytes = B.hq_lss_workspace_bytes(N, C, D)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=device)
        self.probs = torch.empty(max(N, 1), dtype=torch.float64, device=device)
        self.kept_idx = torch.empty(max(N, 1), dtype=torch.int32, device=device)
        self.stats = torch.zeros(4, dtype=torch.int32, device=device)   # one hq_lss_stats

    def __call__(self, dy, saved_x, uniforms, dw, budget, stream=None):
        B.check(B.hq_lss_bwd_weight(
            ptr(dy), HQ_DT[dy.dtype], saved_x.st, self.N, self.C, self.D, self.cfg, float(budget),
            ptr(uniforms), ptr(dw), HQ_DT[dw.dtype], ptr(self.probs), ptr(self.kept_idx),
            ptr(self.stats), ptr(self.ws), self.ws_bytes, stream_ptr(stream)),
            "hq_lss_bwd_weight")

    def read_stats(self):
        """(kept, s8, s_hi, s_lo) on the host."""
        h = self.stats.cpu().numpy()
        f = h.view(np.float32)
        return int(h[0]), np.float32(f[1]), np.float32(f[2]), np.float32(f[3])
