"""Seeded synthetic inputs for the INT8 W8A8 linear layer.

This module only draws random tensors; it holds none of the layer's arithmetic
(no rotation, quantization or products) and serves the oracle tests, the GPU
parity tests and the benchmark alike.  bf16 tensors are returned as uint16 bit
patterns produced by a round-to-nearest-even cast from fp32.

Workloads (shapes and distributions of the layer as used in the pages'
measurements, OneTrainer PR #1681 commit note 1: 5376 -> 7168 at 2048 and
12000 tokens):
  tiny    X fp32 [64,256] ~N(0,1), W [128,256] ~N(0,0.05), b [128] ~N(0,0.01),
          dY fp32 [64,128] ~N(0,1), SGD lr 1e-3, no rotation, seed 0.
  linear  X bf16 [M,K] ~N(0,1) with round(1% of K) channels of a seeded
          permutation scaled x8 before the cast; W [N,K] ~N(0,0.02); dY bf16
          [M,N] ~N(0,0.01).  5376 -> 7168 at M = 2048 (forward) and 12000
          (forward + backward); rotation block 128.
  skinny  M in {1,4,16}, 4096 -> 4096, X bf16 ~N(0,1), W ~N(0,0.02), no
          rotation, no outliers.
  mlp     X bf16 [8192,4096] ~N(0,1), W1 [14336,4096], W2 [4096,14336]
          ~N(0,0.02), dY2 bf16 [8192,4096] ~N(0,0.01), rotation block 128 on
          both inputs, SGD lr 1e-3 with seeds 0 (fc1) and 1 (fc2).
          Per-layer steps of the MLP draw, after those: H [8192,14336] ~N(0,1)
          whose erf-GELU (float64, rounded to fp32) stands in for fc2's input,
          and dY1 fp32 [8192,14336] ~N(0,0.01) for the gradient reaching fc1
          through the GELU.  The GELU sits outside the INT8 path; these inputs
          let each layer be checked on its own at the MLP's shapes.
Draw order is fixed: X, outlier permutation, W, bias, dY.
"""
import math

import numpy as np

HEADLINE = dict(M=12000, K=5376, N=7168, had_block=128)
FORWARD_2048 = dict(M=2048, K=5376, N=7168, had_block=128)


def f32_to_bf16_bits(x):
    """Round-to-nearest-even cast of finite fp32 values to bf16 bit patterns."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def tiny(seed=0):
    rng = np.random.default_rng(seed)
    x = _normal(rng, (64, 256), 1.0)
    w = _normal(rng, (128, 256), 0.05)
    b = _normal(rng, (128,), 0.01)
    dy = _normal(rng, (64, 128), 1.0)
    return dict(x=x, w=w, b=b, dy=dy, lr=1e-3, had_block=0, seed=0)


def linear(M, K, N, *, outliers=True, w_std=0.02, dy_std=0.01, with_dy=True,
           with_bias=False, x_bf16=True, dy_bf16=True, had_block=128, seed=0):
    """Inputs for one linear layer of shape M tokens x K -> N."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, K), 1.0)
    n_out = int(round(0.01 * K)) if outliers else 0
    if n_out:
        chans = rng.permutation(K)[:n_out]
        x[:, chans] *= np.float32(8.0)
    w = _normal(rng, (N, K), w_std)
    b = _normal(rng, (N,), 0.01) if with_bias else None
    dy = _normal(rng, (M, N), dy_std) if with_dy else None
    out = dict(x=f32_to_bf16_bits(x) if x_bf16 else x, w=w, b=b, had_block=had_block,
               seed=seed, outlier_channels=n_out)
    if dy is not None:
        out["dy"] = f32_to_bf16_bits(dy) if dy_bf16 else dy
    return out


def skinny(M, K=4096, N=4096, seed=0):
    return linear(M, K, N, outliers=False, with_dy=False, had_block=0, seed=seed)


def mlp(M=8192, d=4096, h=14336, seed=0):
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, d), 1.0)
    w1 = _normal(rng, (h, d), 0.02)
    w2 = _normal(rng, (d, h), 0.02)
    dy2 = _normal(rng, (M, d), 0.01)
    return dict(x=f32_to_bf16_bits(x), w1=w1, w2=w2, dy2=f32_to_bf16_bits(dy2),
                lr=1e-3, had_block=128, seeds=(0, 1))


def _gelu(h):
    """Exact (erf) GELU, in float64, rounded once to fp32."""
    from scipy.special import erf
    h64 = h.astype(np.float64)
    return (0.5 * h64 * (1.0 + erf(h64 / math.sqrt(2.0)))).astype(np.float32)


def mlp_layer(which, M=8192, d=4096, h=14336, seed=0):
    """Inputs for one layer of the MLP on its own: which = 1 (fc1, d -> h, bf16
    input, fp32 gradient) or 2 (fc2, h -> d, fp32 GELU-output input, bf16
    gradient)."""
    base = mlp(M, d, h, seed)
    rng = np.random.default_rng([seed, 5])
    hid = _normal(rng, (M, h), 1.0)
    if which == 1:
        dy1 = _normal(rng, (M, h), 0.01)
        return dict(x=base["x"], w=base["w1"], b=None, dy=dy1, lr=base["lr"], had_block=128,
                    seed=base["seeds"][0])
    return dict(x=_gelu(hid), w=base["w2"], b=None, dy=base["dy2"], lr=base["lr"],
                had_block=128, seed=base["seeds"][1])
