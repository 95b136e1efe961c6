"""Seeded synthetic inputs for the DiT linear-layer workloads.

This module only draws random tensors and rounds them to bf16 once; it holds
none of the quantization or GEMM arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it.

The pages measure whole-model latency of FLUX.2 [dev] / FLUX 3 Image Klein at
1024x1024 and 2048x2048 ([P2] time-breakdown paragraph) and give no tensor
shapes.  The stand-ins are DiT linear shapes: hidden size 3072, MLP ratio 4,
4096 / 16384 image tokens plus 512 text tokens, batch 2 for a CFG pair.
Activations are N(0,1) (with rare outliers) or Student-t(3) heavy-tailed;
weights are 0.02 * N(0,1).  One ``numpy.random.Generator(PCG64(seed))`` per
workload, seed 0 by default; tensors are drawn in the order listed, as
float32, then rounded to bf16 nearest-even.

Every array returned is a uint16 array of bf16 bit patterns.
"""

import numpy as np

HIDDEN = 3072
MLP = 4 * HIDDEN


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def normal(rng, shape, std=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def student_t3(rng, shape):
    return f32_to_bf16_bits(rng.standard_t(3, size=shape).astype(np.float32))


def normal_with_outliers(rng, shape, frac=0.001, factor=50.0):
    """N(0,1) with round(frac * numel) entries, drawn without replacement, times factor."""
    x = rng.standard_normal(shape, dtype=np.float32)
    n = int(round(frac * x.size))
    idx = rng.choice(x.size, n, replace=False)
    flat = x.reshape(-1)
    flat[idx] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def linear_small(seed=0):
    """Single NVFP4 linear: X [128,1024] ~ N(0,1), W [1024,1024] ~ 0.02 N(0,1)."""
    rng = _rng(seed)
    return {"x": normal(rng, (128, 1024)), "w": normal(rng, (1024, 1024), 0.02)}


def quantize_act(seed=0, rows=16896, cols=HIDDEN):
    """Activation [16896, 3072] (16384 image + 512 text tokens), N(0,1), 0.1% outliers x50."""
    rng = _rng(seed)
    return {"x": normal_with_outliers(rng, (rows, cols))}


def qkv_1024(seed=0):
    """Joint-attention QKV at 1024^2: X [4608,3072] ~ N(0,1), W [9216,3072] ~ 0.02 N(0,1)."""
    rng = _rng(seed)
    return {"x": normal(rng, (4608, HIDDEN)), "w": normal(rng, (3 * HIDDEN, HIDDEN), 0.02)}


def mlp_2048(seed=0, tokens=16896):
    """DiT MLP at 2048^2: X [16896,3072] ~ t(3); W_up [12288,3072], W_down [3072,12288] ~ 0.02 N."""
    rng = _rng(seed)
    return {"x": student_t3(rng, (tokens, HIDDEN)),
            "w_up": normal(rng, (MLP, HIDDEN), 0.02),
            "w_down": normal(rng, (HIDDEN, MLP), 0.02)}


def dit_block_2048(seed=0, tokens=33792):
    """Full DiT-block linear sequence, batch 2 at 2048^2 (M = 33792)."""
    rng = _rng(seed)
    return {"x_qkv": normal(rng, (tokens, HIDDEN)),
            "x_o": normal(rng, (tokens, HIDDEN)),
            "x_mlp": student_t3(rng, (tokens, HIDDEN)),
            "w_qkv": normal(rng, (3 * HIDDEN, HIDDEN), 0.02),
            "w_o": normal(rng, (HIDDEN, HIDDEN), 0.02),
            "w_up": normal(rng, (MLP, HIDDEN), 0.02),
            "w_down": normal(rng, (HIDDEN, MLP), 0.02),
            "temb": normal(rng, (2, HIDDEN)),
            "w_mod": normal(rng, (6 * HIDDEN, HIDDEN), 0.02)}


def random_matrix(seed, shape, kind="normal", std=1.0):
    """Generic seeded matrix for parity cases of arbitrary shape."""
    rng = _rng(seed)
    if kind == "normal":
        return normal(rng, shape, std)
    if kind == "t3":
        return student_t3(rng, shape)
    if kind == "outliers":
        return normal_with_outliers(rng, shape)
    raise ValueError(kind)
