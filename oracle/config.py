"""TurboQuantConfig arithmetic (oracle; test infrastructure only).

Source: vLLM API page "vllm.model_executor.layers.quantization.turboquant",
class ``TurboQuantConfig``: the class docstring (named presets, argument
meanings), the dataclass fields, and the properties ``key_fp8``, ``mse_bits``,
``key_mse_bits``, ``centroid_bits``, ``n_centroids``, ``key_packed_size``,
``effective_value_quant_bits``, ``value_packed_size``, ``slot_size``,
``slot_size_aligned`` and the static method ``from_cache_dtype``.

Pins: slot sizes against the sizes the printed formulas give at head_dim 128
and the two compression ratios of the docstring that agree with them (2.6x,
3.8x); preset fields against the docstring's preset descriptions; the error
text against ``from_cache_dtype``'s message. See tests/test_oracle_config.py.

Bit-width variants: the article on the TurboQuant project's full_tq mode
(section on the next directions, directions 2 and 3) describes 2-bit values
(its value quantizer switches between 2 and 4 bits) and layer-adaptive key bits
(an ``initial_layers_key_bits`` hook parameter that gives the first four layers
one more key bit). The printed size formulas take any bit width, so a 2-bit
value field is ceil(D * 2 / 8) + 4 bytes; ``layer_config`` gives the per-layer
config. Pins: slot sizes by the printed formulas, the layer rule by cases.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

# Preset names and their fields, in the order the class docstring lists them.
# The docstring describes each preset in words: k8v4 = FP8 keys + 4-bit values;
# 4bit_nc = 4-bit MSE keys + 4-bit values + norm correction; k3v4_nc = 3-bit
# MSE keys + 4-bit values + NC; 3bit_nc = 3-bit MSE keys + 3-bit values + NC.
PRESETS = {
    "turboquant_k8v4": (8, 4, False),
    "turboquant_4bit_nc": (4, 4, True),
    "turboquant_k3v4_nc": (3, 4, True),
    "turboquant_3bit_nc": (3, 3, True),
}

DEFAULT_SEED = 42  # dataclass field default


@dataclass(frozen=True)
class TQConfig:
    """The five dataclass fields and the derived properties, as printed."""

    head_dim: int = 128
    key_quant_bits: int = 3
    value_quant_bits: int = 4
    seed: int = DEFAULT_SEED
    norm_correction: bool = False

    # FP8 keys are selected by key_quant_bits == 8 (no rotation, no MSE).
    @property
    def key_fp8(self) -> bool:
        return self.key_quant_bits == 8

    # MSE bit width; in FP8 mode it falls back to the value bit width
    # (centroids are still generated there).
    @property
    def mse_bits(self) -> int:
        return self.value_quant_bits if self.key_fp8 else self.key_quant_bits

    @property
    def key_mse_bits(self) -> int:
        return 0 if self.key_fp8 else self.key_quant_bits

    @property
    def centroid_bits(self) -> int:
        return self.mse_bits

    @property
    def n_centroids(self) -> int:
        return 2 ** self.mse_bits

    # Key field: D bytes in FP8 mode; otherwise the packed MSE indices
    # (ceil(D * bits / 8) bytes) followed by an fp16 vector norm.
    @property
    def key_packed_size(self) -> int:
        if self.key_fp8:
            return self.head_dim
        return math.ceil(self.head_dim * self.key_mse_bits / 8) + 2

    @property
    def effective_value_quant_bits(self) -> int:
        return self.value_quant_bits

    # Value field: packed codes plus an fp16 scale and an fp16 zero.
    @property
    def value_packed_size(self) -> int:
        return math.ceil(self.head_dim * self.value_quant_bits / 8) + 4

    # One slot per head per position: [key_packed | value_packed].
    @property
    def slot_size(self) -> int:
        return self.key_packed_size + self.value_packed_size

    # Rounded up to an even number of bytes.
    @property
    def slot_size_aligned(self) -> int:
        s = self.slot_size
        return s + (s % 2)

    # Not on the pages: the block length of the blockwise Walsh-Hadamard
    # transform, i.e. the largest power of two dividing head_dim (the reading
    # taken for head_dim 96, which the docstring lists as an example size).
    @property
    def wht_block(self) -> int:
        d = self.head_dim
        return d & (-d)


class UnknownPresetError(ValueError):
    pass


def from_cache_dtype(cache_dtype: str, head_dim: int) -> TQConfig:
    """Config from a named preset; the seed keeps its default.

    An unknown name raises ValueError naming the name and listing the valid
    presets (``from_cache_dtype`` on the API page).
    """
    if cache_dtype not in PRESETS:
        valid = ", ".join(PRESETS.keys())
        raise UnknownPresetError(
            f"Unknown TurboQuant cache dtype: {cache_dtype!r}. Valid presets: {valid}"
        )
    kb, vb, nc = PRESETS[cache_dtype]
    return TQConfig(head_dim=head_dim, key_quant_bits=kb, value_quant_bits=vb,
                    norm_correction=nc)


def layer_seed(seed: int, layer_idx: int) -> int:
    """Per-layer seed: base seed plus 1337 times the layer index (``seed``
    argument description in the class docstring), taken modulo 2**64."""
    return (seed + layer_idx * 1337) % (1 << 64)


# Layer-adaptive key bits (article on the TurboQuant project's full_tq mode,
# direction 3): layers below INITIAL_LAYERS use ``initial_layers_key_bits``
# key bits. Readings: the parameter is the key bit width of those layers and
# defaults to one more than the base width; FP8 keys (8) have no wider MSE
# form, so an FP8 base keeps its keys unless a width is given; everything else
# (value bits, norm correction, base seed) is the base config's. The layer's
# seed still comes from layer_seed(seed, layer_idx).
INITIAL_LAYERS = 4


def layer_config(base: TQConfig, layer_idx: int, initial_layers: int = INITIAL_LAYERS,
                 initial_layers_key_bits: int | None = None) -> TQConfig:
    if layer_idx < 0 or initial_layers < 0:
        raise ValueError("layer_idx and initial_layers must be >= 0")
    if layer_idx >= initial_layers:
        return base
    if initial_layers_key_bits is None:
        if base.key_fp8:
            return base
        initial_layers_key_bits = base.key_quant_bits + 1
    return replace(base, key_quant_bits=initial_layers_key_bits)
