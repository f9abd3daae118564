"""Lloyd-Max centroid table for rotated key coordinates (oracle; test only).

Source: vLLM API page "vllm.model_executor.layers.quantization.turboquant",
``TurboQuantConfig`` docstring (keys use Lloyd-Max scalar quantization after
the rotation) and the ``mse_bits`` / ``n_centroids`` properties (2**mse_bits
centroids).

Reading (the pages do not name the target density): after the randomized
Hadamard rotation a unit vector's coordinates are sums of D random-signed
terms, close to Gaussian with variance 1/D, so the table is the Lloyd-Max
quantizer of N(0, 1/D) with L = 2**mse_bits levels: the standard-normal table
scaled by 1/sqrt(D).

The standard-normal table is found by Lloyd's fixed-point iteration (Lloyd
1957/1982; Max 1960): thresholds are the midpoints of adjacent centroids and
each centroid is the conditional mean of its cell,
E[X | a < X <= b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
Only the positive half is iterated (the density is symmetric) and the negative
half is its mirror, so the table is exactly antisymmetric. float64 throughout;
the fp32 table is the rounding of the float64 one, and each fp32 midpoint is
the rounding of the float64 mean of two adjacent float64 centroids.

Pins: Max's published table for N(0,1) at 4, 8 and 16 levels (tests/golden);
the centroid and midpoint conditions checked with scipy quadrature; the
distortion against Max's published mean-squared errors.
"""

from __future__ import annotations

import math

import numpy as np

LLOYD_ITERATIONS = 2000


def _cell_mean(a: float, b: float) -> float:
    """Mean of a standard normal restricted to (a, b], 0 <= a < b <= inf."""
    phi_a = math.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)
    phi_b = 0.0 if math.isinf(b) else math.exp(-0.5 * b * b) / math.sqrt(2.0 * math.pi)
    # Phi(b) - Phi(a) via erfc, which stays accurate in the upper tail.
    erfc_a = math.erfc(a / math.sqrt(2.0))
    erfc_b = 0.0 if math.isinf(b) else math.erfc(b / math.sqrt(2.0))
    return (phi_a - phi_b) / (0.5 * (erfc_a - erfc_b))


def standard_normal_table(levels: int) -> np.ndarray:
    """Lloyd-Max reconstruction levels for N(0,1), ascending, float64."""
    assert levels >= 2 and levels % 2 == 0
    half = levels // 2
    c = [(k + 0.5) * 3.0 / half for k in range(half)]  # positive half, initial guess
    for _ in range(LLOYD_ITERATIONS):
        edges = [0.0] + [(c[k - 1] + c[k]) / 2.0 for k in range(1, half)] + [math.inf]
        c = [_cell_mean(edges[k], edges[k + 1]) for k in range(half)]
    pos = np.array(c, dtype=np.float64)
    return np.concatenate([-pos[::-1], pos])


def centroids_f64(head_dim: int, mse_bits: int) -> np.ndarray:
    """Lloyd-Max levels for N(0, 1/head_dim), float64, ascending."""
    return standard_normal_table(2 ** mse_bits) / math.sqrt(head_dim)


def tables_f32(head_dim: int, mse_bits: int) -> tuple[np.ndarray, np.ndarray]:
    """(centroids fp32 [L], midpoints fp32 [L-1]) as the encoder uses them."""
    c64 = centroids_f64(head_dim, mse_bits)
    c32 = c64.astype(np.float32)
    m32 = ((c64[:-1] + c64[1:]) / 2.0).astype(np.float32)
    return c32, m32
