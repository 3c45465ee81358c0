"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module draws random tensors and nothing else: it holds none of the
quantization arithmetic. Every tensor is returned as bf16 bit patterns
(``numpy.uint16``), made by drawing binary32 values with numpy's PCG64
``default_rng(seed)`` and rounding them to bf16 (nearest, ties to even).

Workload shapes follow the Llama-3-8B MLP at sequence length 8192 (hidden
4096, intermediate 14336) that the NVFP4 MaxText measurement uses (page
"Melatih model dalam 4 bit", section "Angka yang dilaporkan"); the value
distributions are the ones the workload table states (Gaussian activations
with outlier columns, Gaussian weights, Laplace gradients with outliers).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "activation_small",
    "activation",
    "weight",
    "gradient",
    "gemm_operands",
    "gemm_sample_rows",
    "rht_sign_mask",
    "normal_tensor",
    "large_tensor",
    "SR_SEED",
]

# Seed of the stochastic-rounding generator in the gradient workload.
SR_SEED = 42


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bf16 (nearest, ties to even); finite input."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to binary32."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32
    )


def normal_tensor(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    """Plain N(0, std^2) bf16 tensor."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def activation_small(rows: int = 256, cols: int = 1024, seed: int = 0) -> np.ndarray:
    """N(0,1) with 0.1% of the entries (chosen without replacement after the
    bulk draw) multiplied by 50: the small round-trip workload."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(rows * cols, dtype=np.float32)
    k = (rows * cols) // 1000
    idx = rng.choice(rows * cols, size=k, replace=False)
    x[idx] *= np.float32(50.0)
    return f32_to_bf16_bits(x.reshape(rows, cols))


def activation(rows: int = 8192, cols: int = 4096, seed: int = 1, n_outlier_cols: int = 8) -> np.ndarray:
    """Activation (tokens x hidden): N(0,1) with a few random columns
    multiplied by 100."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    cols_idx = rng.choice(cols, size=min(n_outlier_cols, cols), replace=False)
    x[:, cols_idx] *= np.float32(100.0)
    return f32_to_bf16_bits(x)


def weight(rows: int = 14336, cols: int = 4096, seed: int = 2) -> np.ndarray:
    """Weight: i.i.d. N(0, 0.02^2)."""
    return normal_tensor(rows, cols, seed, std=0.02)


def gradient(rows: int = 8192, cols: int = 14336, seed: int = 3) -> np.ndarray:
    """Output gradient: Laplace(0, 1e-3) with 1% of the entries (chosen
    without replacement after the bulk draw) multiplied by 1e3."""
    rng = np.random.default_rng(seed)
    x = rng.laplace(0.0, 1e-3, size=rows * cols).astype(np.float32)
    k = (rows * cols) // 100
    idx = rng.choice(rows * cols, size=k, replace=False)
    x[idx] *= np.float32(1e3)
    return f32_to_bf16_bits(x.reshape(rows, cols))


def gemm_operands(m: int = 8192, n: int = 14336, k: int = 4096, seed_a: int = 4, seed_b: int = 5):
    """A [m][k] ~ N(0,1) (1D-scaled operand) and B [n][k] ~ N(0, 0.02^2)
    (2D-scaled weight operand)."""
    return normal_tensor(m, k, seed_a), normal_tensor(n, k, seed_b, std=0.02)


def gemm_sample_rows(m: int = 8192, count: int = 256, seed: int = 6) -> np.ndarray:
    """Rows of the product the oracle checks in full."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(m, size=min(count, m), replace=False)).astype(np.int64)


def rht_sign_mask(seed: int = 7) -> int:
    """The 16 random signs of the Hadamard transform's diagonal, as a mask
    (bit j set = flip element j of each 16-point segment)."""
    rng = np.random.default_rng(seed)
    return int(rng.integers(0, 1 << 16))


def large_tensor(rows: int = 65552, cols: int = 32768, seed: int = 9) -> np.ndarray:
    """A tensor past 2^31 elements (65552 x 32768 = 2^31 + 2^19, 4.3 GB of
    bf16), built in one pass: row r is row r % 16 of a seeded N(0,1) block
    with its exponent field moved by a seeded per-row shift in [-3, 3]
    (an exact power-of-two rescaling; elements with exponent fields outside
    9..239 are left as drawn). Blocks therefore differ from row to row in
    scale, and every element past offset 2^31 is a distinct function of
    (row, column)."""
    rng = np.random.default_rng(seed)
    base = f32_to_bf16_bits(rng.standard_normal((16, cols), dtype=np.float32))
    shift = rng.integers(-3, 4, size=rows)
    exp_field = (base >> 7) & 0xFF
    movable = (exp_field > 8) & (exp_field < 240)
    table = np.empty((16 * 7, cols), np.uint16)
    for k in range(7):
        moved = (base.astype(np.int32) + ((k - 3) << 7)).astype(np.uint16)
        table[k::7] = np.where(movable, moved, base)
    index = (np.arange(rows) % 16) * 7 + (shift + 3)
    return table[index]
