"""Seeded random signs and the Walsh-Hadamard rotation (oracle; test only).

Source: vLLM API page "vllm.model_executor.layers.quantization.turboquant",
``TurboQuantConfig`` docstring: keys are rotated by a Walsh-Hadamard transform
before Lloyd-Max scalar quantization, the random matrix is generated
deterministically from a base seed, and each layer uses the base seed plus
1337 times its layer index.

Readings (the pages leave these open):

* The rotation is the randomized Hadamard transform
  ``Pi = (1/sqrt(B)) * H_B * diag(s)`` applied blockwise: ``s`` is a vector of
  random signs, ``H_B`` the Sylvester Hadamard matrix in natural order, and
  ``B`` the largest power of two dividing head_dim (B = D for 64 and 128,
  B = 32 for 96, three independent blocks).
* The random signs come from SplitMix64 (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014; output function
  as in S. Vigna's public-domain reference) seeded with the layer seed:
  sign j is -1 when bit 63 of the j-th output is set, else +1.
* The fp32 transform is the in-place butterfly with strides h = 1, 2, 4, ...,
  B/2, each pair (z_j, z_{j+h}) with (j & h) == 0 becoming
  (z_j + z_{j+h}, z_j - z_{j+h}) in round-to-nearest fp32.

Pins: SplitMix64 against published first outputs; the butterfly against
``scipy.linalg.hadamard``; orthogonality and round trip in float64.
"""

from __future__ import annotations

import numpy as np

from .config import layer_seed

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def splitmix64(seed: int, n: int) -> list[int]:
    """First n outputs of SplitMix64 started from state ``seed``."""
    state = seed & _MASK64
    out = []
    for _ in range(n):
        state = (state + _GOLDEN_GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def signs(seed: int, layer_idx: int, head_dim: int) -> np.ndarray:
    """Random signs s_j in {-1, +1} (float32) for one layer."""
    outs = splitmix64(layer_seed(seed, layer_idx), head_dim)
    return np.array([-1.0 if (z >> 63) & 1 else 1.0 for z in outs], dtype=np.float32)


def wht_block(head_dim: int) -> int:
    """Largest power of two dividing head_dim."""
    return head_dim & (-head_dim)


def butterfly_f32(z: np.ndarray, block: int) -> np.ndarray:
    """Unnormalised Sylvester Walsh-Hadamard transform of each length-``block``
    segment of the last axis, fp32, strides ascending (see module header)."""
    z = np.array(z, dtype=np.float32, copy=True)
    lead = z.shape[:-1]
    d = z.shape[-1]
    assert d % block == 0
    h = 1
    while h < block:
        v = z.reshape(*lead, d // (2 * h), 2, h)
        a = v[..., 0, :]
        b = v[..., 1, :]
        z = np.stack([a + b, a - b], axis=-2).reshape(*lead, d)
        h *= 2
    return z


def butterfly_f64(z: np.ndarray, block: int) -> np.ndarray:
    """The same transform in float64 (for the exact-arithmetic identities)."""
    z = np.array(z, dtype=np.float64, copy=True)
    lead = z.shape[:-1]
    d = z.shape[-1]
    h = 1
    while h < block:
        v = z.reshape(*lead, d // (2 * h), 2, h)
        a = v[..., 0, :]
        b = v[..., 1, :]
        z = np.stack([a + b, a - b], axis=-2).reshape(*lead, d)
        h *= 2
    return z


def rotate_f64(x: np.ndarray, s: np.ndarray, block: int) -> np.ndarray:
    """Pi x = (1/sqrt(B)) H_B (s * x), float64, blockwise."""
    return butterfly_f64(np.asarray(x, np.float64) * s.astype(np.float64), block) / np.sqrt(block)


def unrotate_f64(y: np.ndarray, s: np.ndarray, block: int) -> np.ndarray:
    """Pi^T y = s * ((1/sqrt(B)) H_B y): H_B is symmetric and H_B H_B = B I."""
    return s.astype(np.float64) * (butterfly_f64(y, block) / np.sqrt(block))
