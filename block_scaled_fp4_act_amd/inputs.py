"""Seeded synthetic inputs for the residue-compensated FP4 linear.

This module only draws random numbers and shapes them; it holds none of the
quantization or linear arithmetic.  Both the CPU oracle and the HIP path take
their inputs from here, so they see the same values.

Recipe (the workloads of the residue-compensated decode linear, with synthetic
data standing in for captured model activations):
  * W[N, K] fp32 ~ N(0, 0.02^2), drawn with numpy Generator(PCG64(seed)).
  * x[M, K] fp32 ~ N(0, 1); a fixed random set of round(p * K) channels
    (drawn once per workload, shared by every row) is multiplied by a factor.
  * Optionally x is rounded to bf16 (round-to-nearest-even) before quantization.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


def weights(N: int, K: int, seed: int, sigma: float = 0.02) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def outlier_channels(K: int, frac: float, seed: int) -> np.ndarray:
    n = int(round(frac * K))
    g = np.random.Generator(np.random.PCG64(seed))
    return np.sort(g.choice(K, size=n, replace=False))


def activations(M: int, K: int, seed: int, outlier_frac: float, outlier_scale: float,
                outlier_seed: int, bf16: bool) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((M, K), dtype=np.float32)
    ch = outlier_channels(K, outlier_frac, outlier_seed)
    x[:, ch] *= np.float32(outlier_scale)
    if bf16:
        x = round_to_bf16(x)
    return x


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 -> fp32 with round-to-nearest-even (torch's conversion)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


@dataclass(frozen=True)
class Workload:
    name: str
    fmt: str                 # "nvfp4" or "mxfp4"
    M: int
    K: int
    N: int
    w_seed: int
    x_seed: int
    o_seed: int
    outlier_frac: float
    outlier_scale: float
    bf16: bool
    x_rows: int = 0          # rows drawn (M values are prefixes of one draw); 0 -> M

    def draw_x(self) -> np.ndarray:
        rows = self.x_rows or self.M
        x = activations(rows, self.K, self.x_seed, self.outlier_frac, self.outlier_scale,
                        self.o_seed, self.bf16)
        return np.ascontiguousarray(x[: self.M])

    def draw_w(self) -> np.ndarray:
        return weights(self.N, self.K, self.w_seed)

    def with_m(self, M: int) -> "Workload":
        return Workload(self.name, self.fmt, M, self.K, self.N, self.w_seed, self.x_seed,
                        self.o_seed, self.outlier_frac, self.outlier_scale, self.bf16,
                        self.x_rows)


# The five workloads: a small case, the attention projection, an MLP pair, a
# large-MLP M sweep and an MXFP4 case (shapes and distributions as stated).
SMALL = Workload("nvfp4_small_m1_k512_n512", "nvfp4", 1, 512, 512, 0, 1, 2, 0.01, 20.0, False)
ATTN = Workload("nvfp4_attn_m4_k4096_n4096", "nvfp4", 4, 4096, 4096, 0, 1, 2, 0.01, 20.0, True)
MLP_UP = Workload("nvfp4_mlp_up_m8_k4096_n14336", "nvfp4", 8, 4096, 14336, 0, 3, 5, 0.005, 30.0, True)
MLP_DOWN = Workload("nvfp4_mlp_down_m8_k14336_n4096", "nvfp4", 8, 14336, 4096, 1, 4, 6, 0.005, 30.0, True)
LARGE_MLP = Workload("nvfp4_large_mlp_k8192_n28672", "nvfp4", 8, 8192, 28672, 0, 1, 2, 0.005, 30.0, True,
                     x_rows=128)
LARGE_MLP_M = (1, 2, 4, 8, 16, 32, 64, 128)
MX = Workload("mxfp4_k5120_n25600", "mxfp4", 8, 5120, 25600, 0, 1, 2, 0.01, 20.0, True, x_rows=256)
MX_M = (1, 8, 256)

ALL = (SMALL, ATTN, MLP_UP, MLP_DOWN, LARGE_MLP, MX)


# ---- selective compensation (K-Ext) inputs ----
# Channel masks: k of every 8 channels drawn uniformly (bit j of byte g marks
# channel 8g + j).  Calibration rows: fresh draws of a workload's distribution
# (same outlier channels, another seed), standing in for a calibration set.
KEXT_K = (1, 2, 4)           # k = 8 * rho for rho = 0.125, 0.25, 0.5
CALIB_ROWS = 64


def random_masks(K: int, k: int, seed: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    masks = np.zeros((K // 8,), np.uint8)
    for i in range(K // 8):
        for j in g.choice(8, size=k, replace=False):
            masks[i] |= np.uint8(1 << int(j))
    return masks


def calibration_rows(w: Workload, T: int = CALIB_ROWS, seed_offset: int = 1000) -> np.ndarray:
    return activations(T, w.K, w.x_seed + seed_offset, w.outlier_frac, w.outlier_scale, w.o_seed, w.bf16)
