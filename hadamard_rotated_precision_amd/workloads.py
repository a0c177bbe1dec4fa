"""Seeded synthetic inputs for the HQ-MM linear-layer workloads.

This module holds the shapes, distributions and seeds of the five layer workloads and draws
their inputs. It contains none of the method's arithmetic (no rotation, scale, quantization
or product), so both the HIP path and the CPU oracle can take their inputs from here.

Recipe: numpy ``Generator(PCG64(seed))``; values drawn in float64, cast to float32 (RNE),
then rounded RNE to the input dtype (numpy for fp16, a bit-level RNE for bf16). The rounded
bit patterns are what both sides consume. Outlier channels are picked with
``rng.choice(C, n, replace=False)`` after X is drawn and scaled in place.

Layer shapes follow the pages' workloads: a small HQ-MM forward, a HALO-2 step at
2048 x 4096 x 4096, BERT-large FFN-up shapes for the INT4-range learned-step case, the
Llama-7B MLP up/gate layer and a Qwen-14B-shaped down projection.
"""
import math

import numpy as np

F32, F16, BF16 = 0, 1, 2
HALO0, HQ, HALO2 = 0, 1, 2
ABSMAX, STEP = 0, 1
INT, E4M3, E2M3, E3M2 = 0, 1, 2, 3   # code formats (E2M3 / E3M2: FP6)
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}


def lsq_init_step(mean_abs, qp):
    """LSQ-style initial step 2*E|v|/sqrt(Qp) (from the learned-step-size paper, not from
    the pages). Used only to pick a plausible fixed step for the learned-step workload."""
    return float(np.float32(2.0 * mean_abs / math.sqrt(qp)))


def _mean_abs_normal(std):
    return std * math.sqrt(2.0 / math.pi)


# E|T| for Student-t with 3 degrees of freedom = 2*sqrt(3)/pi.
_MEAN_ABS_T3 = 2.0 * math.sqrt(3.0) / math.pi

CONFIGS = {
    1: dict(name="hqmm_fwd_256x512x512_k32", N=256, C=512, D=512, k=32, bits=8,
            mode=ABSMAX, variant=HQ, in_dtype=F16, out_dtype=F32, passes=("fwd",), seed=101,
            x=("normal", 1.0), x_outliers=(4, 50.0), w=("normal", 0.02), dy=None),
    2: dict(name="halo2_2048x4096x4096_k256", N=2048, C=4096, D=4096, k=256, bits=8,
            mode=ABSMAX, variant=HALO2, in_dtype=BF16, out_dtype=BF16,
            passes=("fwd", "dx", "dw"), seed=102,
            x=("normal", 1.0), x_outliers=("frac", 0.001, 100.0), w=("normal", 0.02),
            dy=("t3", 1e-3)),
    3: dict(name="hq_int4step_bert_large_ffn_4096x1024x4096_k16", N=4096, C=1024, D=4096,
            k=16, bits=4, mode=STEP, variant=HQ, in_dtype=F16, out_dtype=F16,
            passes=("fwd", "dx"), seed=103,
            x=("normal", 1.0), x_outliers=(4, 50.0), w=("normal", 0.02), dy=("t3", 1e-3)),
    4: dict(name="halo2_llama7b_mlp_up_4096x4096x11008_k256", N=4096, C=4096, D=11008,
            k=256, bits=8, mode=ABSMAX, variant=HALO2, in_dtype=BF16, out_dtype=BF16,
            passes=("fwd", "dx", "dw"), seed=104,
            x=("t3", 1.0), x_outliers=None, w=("normal", 0.02), dy=("t3", 1e-3)),
    5: dict(name="halo2_qwen14b_down_8192x13824x5120_k128", N=8192, C=13824, D=5120,
            k=128, bits=8, mode=ABSMAX, variant=HALO2, in_dtype=BF16, out_dtype=BF16,
            passes=("fwd", "dx", "dw"), seed=105,
            x=("normal", 1.0), x_outliers=("frac", 0.0005, 200.0), w=("normal", 0.015),
            dy=("lognormal_sign", 1e-3, 1.5)),
}


# Batched products of attention (INT4 page §A.1): the scores S = Q K^T of a Llama-7B-shaped
# attention layer, batch = 4 sequences x 32 heads, 1024 tokens, head_dim 128 (rotated, k = 128),
# HALO-2 (dQ = dS K, dK = dS^T Q). Q and K ~ N(0,1) with 2 head-dim channels x 20 (the outlier
# channels seen in query / key projections); dS = 1e-3 t3.
ATTENTION = {
    "qk": dict(name="halo2_attn_scores_llama7b_128x1024x128x1024_k128", batch=128, N=1024,
               C=128, D=1024, k=128, bits=8, mode=ABSMAX, variant=HALO2, in_dtype=BF16,
               out_dtype=BF16, passes=("fwd", "dx", "dw"), seed=201,
               x=("normal", 1.0), x_outliers=(2, 20.0), w=("normal", 1.0), dy=("t3", 1e-3)),
}


def attention_config(name="qk", **overrides):
    """A copy of a batched (attention) workload; shapes may be overridden."""
    cfg = dict(ATTENTION[name])
    cfg["fmt"] = INT
    cfg.update(overrides)
    return cfg


def make_batched_inputs(cfg):
    """Draw X (batch x N x C), W (batch x D x C) and dY (batch x N x D) for a batched workload,
    as bit arrays of the input dtype; the outlier channels (of C) are shared by all batches
    and by W, as the channels of a head are."""
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    nb, N, C, D = cfg["batch"], cfg["N"], cfg["C"], cfg["D"]
    X = _draw(rng, cfg["x"], (nb, N, C))
    W = _draw(rng, cfg["w"], (nb, D, C))
    outliers = np.zeros(0, dtype=np.int64)
    if cfg.get("x_outliers"):
        n_out, mult = _outlier_count(cfg["x_outliers"], C)
        outliers = rng.choice(C, n_out, replace=False)
        X[:, :, outliers] *= mult
        W[:, :, outliers] *= mult
    dY = _draw(rng, cfg["dy"], (nb, N, D))
    dt = cfg["in_dtype"]
    return dict(x=to_dtype_bits(X, dt), w=to_dtype_bits(W, dt), dy=to_dtype_bits(dY, dt),
                outliers=outliers)


def config(cfg_id, **overrides):
    """A copy of a workload definition; shape keys (N, C, D) may be overridden to draw a
    smaller tensor with the same distributions, and fmt=E4M3 / E2M3 / E3M2 gives the same layer
    with FP8 or FP6 codes (its name then says fp8, fp6e2m3 or fp6e3m2; FP6 codes are 6 bits)."""
    cfg = dict(CONFIGS[cfg_id])
    cfg["id"] = cfg_id
    cfg["fmt"] = INT
    cfg.update(overrides)
    if cfg["fmt"] != INT:
        if CONFIGS[cfg_id]["bits"] != 8 or cfg["mode"] != ABSMAX:
            raise ValueError("float codes are defined for the 8-bit absmax workloads")
        tag = {E4M3: "fp8", E2M3: "fp6e2m3", E3M2: "fp6e3m2"}[cfg["fmt"]]
        cfg["bits"] = 8 if cfg["fmt"] == E4M3 else 6
        base = CONFIGS[cfg_id]["name"]
        cfg["name"] = base.replace("halo2_", "halo2_%s_" % tag).replace("hqmm_", "hqmm_%s_" % tag)
    return cfg


def f32_to_bf16_bits(a):
    """Round float32 to bf16 (RNE) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def to_dtype_bits(a64, dtype):
    """float64 -> float32 (RNE) -> target dtype; fp16/bf16 come back as uint16 bit arrays."""
    a32 = np.asarray(a64, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return a32
    if dtype == F16:
        return a32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return f32_to_bf16_bits(a32)
    raise ValueError("bad dtype")


def _draw(rng, spec, shape):
    kind = spec[0]
    if kind == "normal":
        return rng.standard_normal(shape) * spec[1]
    if kind == "t3":
        return rng.standard_t(3, size=shape) * spec[1]
    if kind == "lognormal_sign":
        mag = np.exp(math.log(spec[1]) + spec[2] * rng.standard_normal(shape))
        sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        return mag * sign
    raise ValueError(kind)


def _outlier_count(spec, C):
    if spec[0] == "frac":
        return max(1, int(round(spec[1] * C))), spec[2]
    return int(spec[0]), float(spec[1])


def make_inputs(cfg):
    """Draw X (N x C), W (D x C) and dY (N x D, or None) for a workload definition.
    Returns dict with 'x', 'w', 'dy' as bit arrays of cfg['in_dtype'], the outlier channel
    indices, and 'steps' (fixed learned-step values) for STEP-mode workloads."""
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    N, C, D = cfg["N"], cfg["C"], cfg["D"]
    X = _draw(rng, cfg["x"], (N, C))
    outliers = np.zeros(0, dtype=np.int64)
    n_out, mult = 0, 1.0
    if cfg.get("x_outliers"):
        n_out, mult = _outlier_count(cfg["x_outliers"], C)
        outliers = rng.choice(C, n_out, replace=False)
        X[:, outliers] *= mult
    W = _draw(rng, cfg["w"], (D, C))
    dY = _draw(rng, cfg["dy"], (N, D)) if cfg.get("dy") else None
    dt = cfg["in_dtype"]
    out = dict(x=to_dtype_bits(X, dt), w=to_dtype_bits(W, dt),
               dy=None if dY is None else to_dtype_bits(dY, dt), outliers=outliers)
    if cfg["mode"] == STEP:
        out["steps"] = fixed_steps(cfg, n_out, mult)
    return out


def fixed_steps(cfg, n_outliers=0, mult=1.0):
    """Fixed step values for the learned-step workload: the LSQ initialisation applied to the
    expected |entry| of each rotated tensor under the workload's distribution (a +-1-weighted
    sum of k independent entries has std sqrt(k) times theirs; the outlier channels raise the
    variance of the blocks they fall in). These are inputs, like trained parameters."""
    k, C = cfg["k"], cfg["C"]
    qp = 7 if cfg["bits"] == 4 else 127
    rk = k if cfg["variant"] != HALO0 else 1
    # X: blocks of rk channels; fraction of blocks holding one outlier channel.
    sx = cfg["x"][1]
    var_plain = rk * sx * sx
    var_out = (rk - 1) * sx * sx + (mult * sx) ** 2
    frac_out = min(1.0, n_outliers * rk / C)
    mean_abs_x = (1 - frac_out) * _mean_abs_normal(math.sqrt(var_plain)) + \
        frac_out * _mean_abs_normal(math.sqrt(var_out))
    mean_abs_w = _mean_abs_normal(math.sqrt(rk) * cfg["w"][1])
    steps = {"x": lsq_init_step(mean_abs_x, qp), "w": lsq_init_step(mean_abs_w, qp)}
    if cfg.get("dy"):
        if cfg["dy"][0] != "t3":
            raise ValueError("fixed steps defined for t3 gradients only")
        kg = k if cfg["variant"] == HALO2 else 1
        # a +-1 sum of kg t3 entries: mean |.| grows like sqrt(kg) (normal approximation).
        steps["g"] = lsq_init_step(_MEAN_ABS_T3 * cfg["dy"][1] * math.sqrt(kg), qp)
    return steps
