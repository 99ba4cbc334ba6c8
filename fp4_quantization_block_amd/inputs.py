"""Seeded synthetic inputs shaped like the pages' Llama-class layers.

This module only draws random tensors; it holds none of the quantization or
GEMM arithmetic.  The CPU oracle and the HIP path both consume what it
returns.  The pages train OLMo-7B, Llama-2-13B and Llama-3 8B on real data;
no weights or datasets are used here -- these are stand-ins with those
layers' shapes and plausible value distributions.

Recipe: each tensor gets its own numpy PCG64 stream seeded with
SeedSequence([workload_seed, tensor_index]); values are drawn in float64 or
float32 and rounded to bfloat16 by torch on the CPU (round to nearest even).
bf16 tensors are returned as uint16 bit patterns (numpy), fp32 as float32.
"""
from dataclasses import dataclass, field
from typing import Dict, Tuple

import numpy as np
import torch

# Philox key for stochastic rounding in the benchmark and parity runs.
SR_SEED = 0x00C0FFEE5EED0004
SR_OFFSET = 0


def _rng(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (RNE) as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal(seed, index, shape, std=1.0):
    g = _rng(seed, index)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def student_t_with_outlier_channels(seed, index, shape, nu=3.0, frac=0.001, factor=100.0):
    """Student-t(nu) activations; round(frac * cols) seeded columns (K
    channels) multiplied by `factor`."""
    g = _rng(seed, index)
    a = g.standard_t(nu, size=shape).astype(np.float32)
    nout = int(round(frac * shape[1]))
    cols = g.permutation(shape[1])[:nout]
    a[:, cols] *= np.float32(factor)
    return a


def normal_with_outlier_elements(seed, index, shape, p=0.01, factor=50.0):
    """N(0,1) with each element independently (Bernoulli(p)) scaled by `factor`."""
    g = _rng(seed, index)
    a = g.standard_normal(size=shape, dtype=np.float32)
    mask = g.random(size=shape, dtype=np.float32) < p
    a[mask] *= np.float32(factor)
    return a


def laplace(seed, index, shape, b=1e-3):
    g = _rng(seed, index)
    return g.laplace(0.0, b, size=shape).astype(np.float32)


@dataclass
class Workload:
    name: str
    seed: int
    tensors: Dict[str, np.ndarray] = field(default_factory=dict)   # uint16 (bf16) or float32
    meta: Dict[str, object] = field(default_factory=dict)


# Full sizes of the five workloads.
FULL_SHAPES = {
    "mxfp8_gemm_256": {"M": 256, "N": 256, "K": 256},
    "moss_two_level_4096": {"M": 4096, "N": 4096, "K": 4096},
    "llama3_8b_mlp": {"T": 8192, "H": 4096, "F": 14336},
    "mxfp4_wgrad_qkv": {"T": 16384, "H": 4096, "Q": 6144},
    "dual_layout_16384x14336": {"R": 16384, "C": 14336},
    # MOSS weight auto-scaling on the 4096x4096 weight of the two-level
    # workload: this step's weights and gradient, and the page's lr
    "moss_weight_autoscale_4096": {"K": 4096, "N": 4096},
    # COAT optimizer states: Adam's first and second moments of the
    # Llama-3-8B gate-up weight (4096 x 28672), fp32
    "coat_optstate_llama_wgu": {"H": 4096, "F2": 28672},
    "nvfp_llama3_8b_gate": {"T": 8192, "H": 4096, "F": 14336},
}
WORKLOAD_SEEDS = {"mxfp8_gemm_256": 1, "moss_two_level_4096": 2, "llama3_8b_mlp": 3,
                  "mxfp4_wgrad_qkv": 4, "dual_layout_16384x14336": 5,
                  "moss_weight_autoscale_4096": 6, "coat_optstate_llama_wgu": 7,
                  "nvfp_llama3_8b_gate": 8}


def make(name: str, **shape_override) -> Workload:
    """Build a workload's tensors; shape keys may be overridden to make a
    smaller instance with the same distributions."""
    shp = dict(FULL_SHAPES[name])
    shp.update(shape_override)
    seed = WORKLOAD_SEEDS[name]
    w = Workload(name, seed, meta=dict(shp))
    if name == "mxfp8_gemm_256":
        M, N, K = shp["M"], shp["N"], shp["K"]
        w.tensors["A"] = normal(seed, 0, (M, K))                 # fp32 [M][K]
        w.tensors["B"] = normal(seed, 1, (K, N))                 # fp32 [K][N]
    elif name == "moss_two_level_4096":
        M, N, K = shp["M"], shp["N"], shp["K"]
        w.tensors["A"] = to_bf16_bits(student_t_with_outlier_channels(seed, 0, (M, K)))
        w.tensors["B"] = to_bf16_bits(normal(seed, 1, (K, N), std=0.02))
    elif name == "llama3_8b_mlp":
        T, H, F = shp["T"], shp["H"], shp["F"]
        w.tensors["X"] = to_bf16_bits(normal(seed, 0, (T, H)))
        w.tensors["W_gu"] = to_bf16_bits(normal(seed, 1, (H, 2 * F), std=0.02))
        w.tensors["Xp"] = to_bf16_bits(normal(seed, 2, (T, F)))
        w.tensors["W_d"] = to_bf16_bits(normal(seed, 3, (F, H), std=0.02))
        w.tensors["dY_gu"] = to_bf16_bits(normal(seed, 4, (T, 2 * F), std=1e-3))
        w.tensors["dY_d"] = to_bf16_bits(normal(seed, 5, (T, H), std=1e-3))
    elif name == "mxfp4_wgrad_qkv":
        T, H, Q = shp["T"], shp["H"], shp["Q"]
        w.tensors["dY"] = to_bf16_bits(laplace(seed, 0, (T, Q)))
        w.tensors["X"] = to_bf16_bits(laplace(seed, 1, (T, H)))
    elif name == "dual_layout_16384x14336":
        R, C = shp["R"], shp["C"]
        w.tensors["X"] = to_bf16_bits(normal_with_outlier_elements(seed, 0, (R, C)))
    elif name == "moss_weight_autoscale_4096":
        K, N = shp["K"], shp["N"]
        w.tensors["W"] = to_bf16_bits(normal(seed, 0, (K, N), std=0.02))     # like the MOSS weight B
        w.tensors["G"] = to_bf16_bits(normal(seed, 1, (K, N), std=1e-3))     # like the MLP gradients
        w.meta["lr"] = 1e-3
    elif name == "nvfp_llama3_8b_gate":
        # Llama-3-8B gate projection, forward: activations with outlier
        # channels (as the MOSS workload), weights N(0, 0.02^2); Y = X W
        T, H, F = shp["T"], shp["H"], shp["F"]
        w.tensors["X"] = to_bf16_bits(student_t_with_outlier_channels(seed, 0, (T, H)))
        w.tensors["W"] = to_bf16_bits(normal(seed, 1, (H, F), std=0.02))
    elif name == "coat_optstate_llama_wgu":
        H, F2 = shp["H"], shp["F2"]
        # first moment: signed, N(0, 1e-3) (max/min within a 128-group of
        # order 1e3, the page's figure); second moment: positive,
        # log-normal 1e-6 * exp(N(0, 0.5)) (max/min of order 10)
        w.tensors["m"] = normal(seed, 0, (H, F2), std=1e-3)
        g = _rng(seed, 1)
        w.tensors["v"] = (np.exp(g.standard_normal(size=(H, F2), dtype=np.float32) * np.float32(0.5))
                          * np.float32(1e-6)).astype(np.float32)
    else:
        raise KeyError(name)
    return w


def sample_blocks(rng: np.random.Generator, rows: int, cols: int, axis: int, n: int,
                  include_corners: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Block start positions (r0, c0) for sampled parity checks; axis 0 = row
    blocks (1x32 along a row), 1 = column blocks (32x1 down a column)."""
    if axis == 0:
        r = rng.integers(0, rows, n)
        c = rng.integers(0, cols // 32, n) * 32
        if include_corners:
            r = np.concatenate([r, [0, 0, rows - 1, rows - 1]])
            c = np.concatenate([c, [0, cols - 32, 0, cols - 32]])
    else:
        r = rng.integers(0, rows // 32, n) * 32
        c = rng.integers(0, cols, n)
        if include_corners:
            r = np.concatenate([r, [0, 0, rows - 32, rows - 32]])
            c = np.concatenate([c, [0, cols - 1, 0, cols - 1]])
    return r.astype(np.int64), c.astype(np.int64)


def sample_tile_entries(rng: np.random.Generator, M: int, N: int, per_tile: int = 16,
                        tile: int = 128) -> Tuple[np.ndarray, np.ndarray]:
    """Output entries (ii, jj) of an M x N matrix for a stratified check: in
    every tile x tile block (ragged edge blocks included) its four corners
    plus per_tile - 4 uniformly drawn entries."""
    ti = np.arange(0, M, tile)
    tj = np.arange(0, N, tile)
    r0 = np.repeat(ti, len(tj))
    c0 = np.tile(tj, len(ti))
    r1 = np.minimum(r0 + tile, M) - 1
    c1 = np.minimum(c0 + tile, N) - 1
    nt = r0.size
    extra = per_tile - 4
    rr = r0[:, None] + (rng.random((nt, extra)) * (r1 - r0 + 1)[:, None]).astype(np.int64)
    cc = c0[:, None] + (rng.random((nt, extra)) * (c1 - c0 + 1)[:, None]).astype(np.int64)
    ii = np.concatenate([np.stack([r0, r0, r1, r1], 1), rr], 1).ravel()
    jj = np.concatenate([np.stack([c0, c1, c0, c1], 1), cc], 1).ravel()
    return ii.astype(np.int64), jj.astype(np.int64)
