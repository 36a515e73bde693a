"""Seeded synthetic inputs for the quantized linear layer (shared by tests, smoke and bench).

This module holds no step of the method: it only draws random tensors, rounds
them to bf16 (round-to-nearest-even) and returns their bit patterns.  It imports
neither the oracle nor the HIP library.

Seeding: ``numpy.random.default_rng([cfg, shape_idx, role, layer, step])`` with
roles W=1, x=2, A=3, B=4, W-outlier choice=5, x-outlier choice=6, dA=7, dB=8.
Values are drawn in float32; outliers multiply whole input channels (columns of
W, columns of x) before the rounding.

The workloads are the five layer configurations this library is measured on:

1. one NVFP4 layer 256x512, x 4x512, LoRA rank 8;
2. decode GEMVs of 7B-class projections, M in {1, 8, 64}, LoRA rank 32;
3. prefill GEMMs of 32B-class MLPs, M = 4096, LoRA rank 64;
4. the FP8 blockwise recipe on an 8B-class MLP, M = 8192;
5. a whole 64-layer 32B-class policy: requantize after a rank-64 update, then a
   decode step at 256 tokens through all 448 linears.
"""

import numpy as np

W_ROLE, X_ROLE, A_ROLE, B_ROLE, WOUT_ROLE, XOUT_ROLE, DA_ROLE, DB_ROLE = range(1, 9)


def rng(cfg, shape_idx, role, layer=0, step=0):
    return np.random.default_rng([cfg, shape_idx, role, layer, step])


def to_bf16_bits(x):
    """finite float32 array -> bf16 bit patterns (uint16), round to nearest even.
    (For finite inputs the 32-bit sum below cannot wrap.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    return (r >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std, g, outlier_frac=0.0, outlier_mult=1.0, out_rng=None):
    """N(0, std) in float32, optional outlier input channels (last axis), rounded to bf16."""
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outlier_frac > 0:
        k = shape[-1]
        cnt = int(round(outlier_frac * k))
        cols = (out_rng if out_rng is not None else g).choice(k, size=cnt, replace=False)
        x[..., cols] *= np.float32(outlier_mult)
    return to_bf16_bits(x)


def student_t_bf16(shape, nu, g):
    """Standard Student-t(nu) draws (heavy-tailed 'N(0,1)-like'), rounded to bf16."""
    return to_bf16_bits(g.standard_t(nu, size=shape).astype(np.float32))


# ------------------------------------------------------------------ configs --

CFG1 = dict(N=256, K=512, M=4, rank=8, lora_scale=2.0, w_std=0.02, w_out=0.01, w_mult=15.0)
CFG2_SHAPES = [(3584, 3584), (3584, 512), (3584, 18944), (18944, 3584)]      # (K, N)
CFG2_M = [1, 8, 64]
CFG2 = dict(rank=32, lora_scale=2.0, w_std=0.02, w_out=0.005, w_mult=20.0)
CFG3_SHAPES = [(5120, 27648), (27648, 5120)]                                  # (K, N)
CFG3 = dict(M=4096, rank=64, lora_scale=2.0, w_std=0.015, w_out=0.005, w_mult=20.0,
            x_out=0.001, x_mult=50.0)
CFG4_SHAPES = [(4096, 14336), (14336, 4096)]                                  # (K, N)
CFG4 = dict(M=8192, nu=3)
# whole policy: per decoder layer (name, K, N)
CFG5_LINEARS = [("q", 5120, 8192), ("k", 5120, 1024), ("v", 5120, 1024), ("o", 8192, 5120),
                ("gate", 5120, 27648), ("up", 5120, 27648), ("down", 27648, 5120)]
CFG5 = dict(layers=64, M=256, rank=32, lora_scale=2.0, w_std=0.015, w_out=0.005, w_mult=20.0,
            delta_rank=64, delta_std=1e-3)


def lora_pair(cfg, shape_idx, k, n, rank, std=0.01, layer=0):
    a = normal_bf16((rank, k), std, rng(cfg, shape_idx, A_ROLE, layer))
    b = normal_bf16((n, rank), std, rng(cfg, shape_idx, B_ROLE, layer))
    return a, b


def config1():
    c = CFG1
    w = normal_bf16((c["N"], c["K"]), c["w_std"], rng(1, 0, W_ROLE), c["w_out"], c["w_mult"],
                    rng(1, 0, WOUT_ROLE))
    x = normal_bf16((c["M"], c["K"]), 1.0, rng(1, 0, X_ROLE))
    a, b = lora_pair(1, 0, c["K"], c["N"], c["rank"])
    return dict(w=w, x=x, a=a, b=b, rank=c["rank"], lora_scale=c["lora_scale"])


def config2_weight(shape_idx):
    k, n = CFG2_SHAPES[shape_idx]
    c = CFG2
    return normal_bf16((n, k), c["w_std"], rng(2, shape_idx, W_ROLE), c["w_out"], c["w_mult"],
                       rng(2, shape_idx, WOUT_ROLE))


def config2_x(shape_idx, m):
    k, _ = CFG2_SHAPES[shape_idx]
    return normal_bf16((m, k), 1.0, rng(2, shape_idx, X_ROLE, step=m))


def config2_lora(shape_idx):
    k, n = CFG2_SHAPES[shape_idx]
    return lora_pair(2, shape_idx, k, n, CFG2["rank"])


def config3_weight(shape_idx):
    k, n = CFG3_SHAPES[shape_idx]
    c = CFG3
    return normal_bf16((n, k), c["w_std"], rng(3, shape_idx, W_ROLE), c["w_out"], c["w_mult"],
                       rng(3, shape_idx, WOUT_ROLE))


def config3_x(shape_idx, m=None):
    k, _ = CFG3_SHAPES[shape_idx]
    c = CFG3
    return normal_bf16((c["M"] if m is None else m, k), 1.0, rng(3, shape_idx, X_ROLE),
                       c["x_out"], c["x_mult"], rng(3, shape_idx, XOUT_ROLE))


def config3_lora(shape_idx):
    k, n = CFG3_SHAPES[shape_idx]
    return lora_pair(3, shape_idx, k, n, CFG3["rank"])


def config4_weight(shape_idx):
    k, n = CFG4_SHAPES[shape_idx]
    return normal_bf16((n, k), 0.02, rng(4, shape_idx, W_ROLE))


def config4_x(shape_idx, m=None):
    k, _ = CFG4_SHAPES[shape_idx]
    return student_t_bf16((CFG4["M"] if m is None else m, k), CFG4["nu"], rng(4, shape_idx, X_ROLE))
