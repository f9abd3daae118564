"""Pins of the oracle's config arithmetic against the printed TurboQuantConfig
code (vLLM API page, TurboQuantConfig properties and from_cache_dtype)."""

import json
import os

import pytest

from oracle import config as C
from tests.conftest import GOLDEN


def _cases():
    with open(os.path.join(GOLDEN, "slot_sizes.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c.get('preset', c.get('bits'))}-d{c['head_dim']}")
def test_slot_sizes_match_printed_formulas(case):
    if "preset" in case:
        cfg = C.from_cache_dtype(case["preset"], case["head_dim"])
    else:
        kb, vb = case["bits"]
        cfg = C.TQConfig(head_dim=case["head_dim"], key_quant_bits=kb, value_quant_bits=vb)
    assert cfg.key_packed_size == case["key"]
    assert cfg.value_packed_size == case["value"]
    assert cfg.slot_size == case["slot"]
    assert cfg.slot_size_aligned == case["aligned"]
    assert cfg.slot_size_aligned % 2 == 0
    if "docstring_ratio" in case:
        # the docstring's ratio is bf16 K+V bytes (4*D) over the slot, to 1 decimal
        assert round(4 * case["head_dim"] / cfg.slot_size_aligned, 1) == case["docstring_ratio"]


def test_docstring_ratios_that_disagree_with_formula():
    # Recorded contradiction: the docstring prints ~3.5x and 4.9x; the formula gives these.
    r1 = 512 / C.from_cache_dtype("turboquant_k3v4_nc", 128).slot_size_aligned
    r2 = 512 / C.from_cache_dtype("turboquant_3bit_nc", 128).slot_size_aligned
    assert round(r1, 2) == 4.34 and round(r2, 2) == 5.02


def test_presets_follow_docstring_descriptions():
    k8 = C.from_cache_dtype("turboquant_k8v4", 128)
    assert k8.key_fp8 and k8.key_quant_bits == 8 and k8.value_quant_bits == 4 and not k8.norm_correction
    n4 = C.from_cache_dtype("turboquant_4bit_nc", 128)
    assert (n4.key_quant_bits, n4.value_quant_bits, n4.norm_correction) == (4, 4, True)
    k3 = C.from_cache_dtype("turboquant_k3v4_nc", 128)
    assert (k3.key_quant_bits, k3.value_quant_bits, k3.norm_correction) == (3, 4, True)
    b3 = C.from_cache_dtype("turboquant_3bit_nc", 128)
    assert (b3.key_quant_bits, b3.value_quant_bits, b3.norm_correction) == (3, 3, True)
    for cfg in (k8, n4, k3, b3):
        assert cfg.seed == 42


def test_derived_properties():
    k8 = C.from_cache_dtype("turboquant_k8v4", 128)
    # FP8 mode: MSE bits fall back to the value bits, key MSE bits are 0
    assert k8.mse_bits == 4 and k8.key_mse_bits == 0 and k8.centroid_bits == 4 and k8.n_centroids == 16
    b3 = C.from_cache_dtype("turboquant_3bit_nc", 128)
    assert b3.mse_bits == 3 and b3.key_mse_bits == 3 and b3.n_centroids == 8
    assert b3.effective_value_quant_bits == 3
    d = C.TQConfig()
    assert (d.head_dim, d.key_quant_bits, d.value_quant_bits, d.seed, d.norm_correction) == (128, 3, 4, 42, False)


def test_unknown_preset_message():
    with pytest.raises(ValueError) as ei:
        C.from_cache_dtype("turboquant_2bit", 128)
    msg = str(ei.value)
    assert msg.startswith("Unknown TurboQuant cache dtype: 'turboquant_2bit'. Valid presets: ")
    assert msg.endswith("turboquant_k8v4, turboquant_4bit_nc, turboquant_k3v4_nc, turboquant_3bit_nc")


def test_layer_seed():
    assert C.layer_seed(42, 0) == 42
    assert C.layer_seed(42, 3) == 42 + 3 * 1337
    assert C.layer_seed(2 ** 64 - 1, 1) == 1336


def test_wht_block():
    assert C.TQConfig(head_dim=128).wht_block == 128
    assert C.TQConfig(head_dim=96).wht_block == 32
    assert C.TQConfig(head_dim=64).wht_block == 64


# ---------------------------------------------------------------- layer-adaptive key bits
# The TurboQuant project article's direction 3: the first four layers get one
# more key bit (initial_layers_key_bits); later layers keep the base config.

@pytest.mark.parametrize("preset,first_kb", [("turboquant_k3v4_nc", 4), ("turboquant_3bit_nc", 4),
                                             ("turboquant_4bit_nc", 5)])
def test_layer_config_first_four_layers_get_one_more_key_bit(preset, first_kb):
    base = C.from_cache_dtype(preset, 128)
    for layer in range(8):
        lc = C.layer_config(base, layer)
        if layer < 4:
            assert lc.key_quant_bits == first_kb
            assert (lc.value_quant_bits, lc.norm_correction, lc.seed, lc.head_dim) == \
                (base.value_quant_bits, base.norm_correction, base.seed, base.head_dim)
        else:
            assert lc == base


def test_layer_config_slot_sizes():
    base = C.from_cache_dtype("turboquant_k3v4_nc", 128)
    # layers 0-3: 4-bit keys -> the 4bit_nc slot (134 B); from layer 4 the k3v4 slot (118 B)
    assert [C.layer_config(base, i).slot_size_aligned for i in range(6)] == [134] * 4 + [118] * 2
    b2 = C.TQConfig(head_dim=128, key_quant_bits=3, value_quant_bits=2, norm_correction=True)
    assert C.layer_config(b2, 0).slot_size_aligned == 102 and C.layer_config(b2, 4).slot_size_aligned == 86


def test_layer_config_fp8_and_explicit_width():
    k8 = C.from_cache_dtype("turboquant_k8v4", 128)
    assert C.layer_config(k8, 0) == k8          # no wider form of FP8 keys
    assert C.layer_config(k8, 0, initial_layers_key_bits=4).key_quant_bits == 4
    base = C.from_cache_dtype("turboquant_3bit_nc", 128)
    assert C.layer_config(base, 1, initial_layers_key_bits=8).key_fp8
    assert C.layer_config(base, 1, initial_layers=0) == base
    assert C.layer_config(base, 5, initial_layers=6).key_quant_bits == 4
    with pytest.raises(ValueError):
        C.layer_config(base, -1)
