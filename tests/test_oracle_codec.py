"""Pins of the oracle's encoders, bit packing, FP8 and dequantization."""

import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import codec as X
from oracle import config as C
from oracle import lloyd_max as LM
from oracle import rotation as R
from tests.conftest import GOLDEN


# ---------------------------------------------------------------- packing

def test_pack_worked_examples():
    with open(os.path.join(GOLDEN, "pack_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        codes = np.array([e["codes"]], dtype=np.uint8)
        got = X.pack_bits(codes, e["bits"])[0].tobytes().hex()
        assert got == e["bytes_hex"], e
        back = X.unpack_bits(X.pack_bits(codes, e["bits"]), e["bits"], codes.shape[1])
        assert np.array_equal(back, codes)


@pytest.mark.parametrize("bits,d", [(3, 128), (4, 128), (3, 96), (4, 64), (3, 64), (2, 128), (2, 96)])
def test_pack_round_trip_and_size(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    codes = rng.integers(0, 2 ** bits, size=(50, d), dtype=np.uint8)
    p = X.pack_bits(codes, bits)
    assert p.shape == (50, math.ceil(d * bits / 8))
    assert np.array_equal(X.unpack_bits(p, bits, d), codes)
    # element j's lowest bit sits at stream bit j*bits
    for j in (0, 1, d - 1):
        bit = j * bits
        assert ((p[:, bit // 8] >> (bit % 8)) & 1 == (codes[:, j] & 1)).all()


# ---------------------------------------------------------------- FP8

def _all_bf16_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


def test_fp8_encode_matches_torch_exhaustively_in_range():
    x = _all_bf16_f32()
    ok = np.isfinite(x) & (np.abs(x) < 464.0)
    x = x[ok]
    ours = X.fp8_e4m3fn_encode(x)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = X.fp8_e4m3fn_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_fp8_specials_and_saturation():
    # (value, code): exact values, ties to even, saturation, signed zero
    cases = [(448.0, 0x7E), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (1.0, 0x38), (1.5 * 2.0 ** -9, 0x02),
             (500.0, 0x7E), (-500.0, 0xFE), (1e30, 0x7E), (float("inf"), 0x7E), (-0.0, 0x80),
             (-(2.0 ** -11), 0x80), (0.0, 0x00), (17.0, 0x58), (18.0, 0x59), (9.0, 0x51), (-9.5, 0xD2)]
    for v, code in cases:
        assert int(X.fp8_e4m3fn_encode(np.array([v], np.float32))[0]) == code, v
    assert int(X.fp8_e4m3fn_encode(np.array([np.nan], np.float32))[0]) & 0x7F == 0x7F


# ---------------------------------------------------------------- values

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_constant_vector(bits):
    v = np.full((3, 64), 0.7, dtype=np.float32)
    codes, s16, z16 = X.encode_values(v, bits)
    assert (codes == 0).all() and (s16 == 0).all()
    assert np.array_equal(z16, np.full(3, np.float16(0.7).view(np.uint16)))
    _, vhat = X.dequant_f32(X.encode_slots(np.ones((3, 64), np.float32), v,
                                           C.TQConfig(head_dim=64, value_quant_bits=bits), 0),
                            C.TQConfig(head_dim=64, value_quant_bits=bits), 0)
    assert np.array_equal(vhat, np.full((3, 64), np.float32(np.float16(0.7))))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_integer_ramp(bits):
    levels = 2 ** bits - 1
    ramp = np.tile(np.arange(levels + 1, dtype=np.float32), 8)[None, :]
    codes, s16, z16 = X.encode_values(ramp, bits)
    assert X.f16_bits_to_f32(s16)[0] == 1.0 and X.f16_bits_to_f32(z16)[0] == 0.0
    assert np.array_equal(codes[0], ramp[0].astype(np.uint8))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_error_bound(bits):
    rng = np.random.default_rng(bits)
    v = (rng.standard_normal((400, 128)) * rng.uniform(0.01, 20, (400, 1))).astype(np.float32)
    codes, s16, z16 = X.encode_values(v, bits)
    s1, z1 = X.f16_bits_to_f32(s16), X.f16_bits_to_f32(z16)
    levels = 2 ** bits - 1
    scale32 = (v.max(1) - v.min(1)) / np.float32(levels)
    vhat = s1[:, None].astype(np.float64) * codes + z1[:, None]
    bound = s1 / 2 + levels * np.abs(scale32 - s1) + np.abs(z1 - v.min(1)) + 1e-6 * np.abs(v).max(1)
    assert (np.abs(vhat - v).max(1) <= bound).all()
    # codes span the full range on generic data
    assert codes.min() == 0 and codes.max() == levels


# ---------------------------------------------------------------- keys

def _cfg(d, kb, vb=4, nc=False, seed=42):
    return C.TQConfig(head_dim=d, key_quant_bits=kb, value_quant_bits=vb, norm_correction=nc, seed=seed)


@pytest.mark.parametrize("d,kb", [(128, 3), (128, 4), (96, 3), (64, 3), (64, 4)])
def test_key_index_is_nearest_centroid_of_explicit_rotation(d, kb):
    """Independent formulation: u = (H diag(s) x) / (sqrt(B) ||x||) with the
    Hadamard matrix from scipy, index = argmin_k |u - c_k| in float64."""
    cfg = _cfg(d, kb)
    rng = np.random.default_rng(d + kb)
    x = rng.standard_normal((300, d)).astype(np.float32)
    x[:, :4] *= 10
    idx, norm16 = X.encode_keys_mse(x, cfg, layer_idx=3)
    blk = cfg.wht_block
    s = R.signs(42, 3, d).astype(np.float64)
    h = scipy.linalg.block_diag(*([scipy.linalg.hadamard(blk)] * (d // blk))).astype(np.float64)
    u = (x.astype(np.float64) * s) @ h.T / (math.sqrt(blk) * np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True))
    c32, m32 = LM.tables_f32(d, kb)
    want = np.abs(u[:, :, None] - c32.astype(np.float64)[None, None, :]).argmin(axis=2)
    near_edge = np.abs(u[:, :, None] - m32.astype(np.float64)[None, None, :]).min(axis=2) < 1e-6
    assert np.array_equal(idx[~near_edge], want[~near_edge])
    assert near_edge.mean() < 1e-3
    # vec_norm within one fp16 ulp of the float64 norm
    n64 = np.linalg.norm(x.astype(np.float64), axis=1)
    n16 = X.f16_bits_to_f32(norm16).astype(np.float64)
    assert (np.abs(n16 - n64) <= np.spacing(np.float16(n64).astype(np.float16)).astype(np.float64)).all()


@pytest.mark.parametrize("kb,expect", [(3, 0.0345), (4, 0.0095)])
def test_key_distortion_matches_lloyd_max_theory(kb, expect):
    """Relative squared error of a dequantized Gaussian key is the Lloyd-Max
    distortion of one standard-normal coordinate (Max 1960)."""
    cfg = _cfg(128, kb)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2000, 128)).astype(np.float32)
    slots = X.encode_slots(x, x, cfg, 0)
    khat, _ = X.dequant_f64(slots, cfg, 0)
    rel = ((khat - x) ** 2).sum(1) / (x.astype(np.float64) ** 2).sum(1)
    assert abs(rel.mean() - expect) / expect < 0.1


@pytest.mark.parametrize("d,kb", [(128, 4), (128, 3), (96, 4), (96, 3), (64, 4), (64, 3)])
def test_key_index_at_midpoint_ties(d, kb):
    """Rotated coordinates exactly on each midpoint m_k, and one fp32 ulp
    above and below it: the index is the number of midpoints strictly below
    u (k on the midpoint, k + 1 above, k below). A >= in place of the strict
    compare, or an off-by-one bin, fails here."""
    from tests.midpoint_keys import rotated_unit, tie_keys
    cfg = _cfg(d, kb)
    keys, cases = tie_keys(cfg, layer_idx=1, seed=d + kb)
    _, m32 = LM.tables_f32(d, kb)
    u = rotated_unit(keys, cfg, 1)
    idx, _ = X.encode_keys_mse(keys, cfg, 1)
    # u in float64 straight from the definition, to check the keys' u
    blk = cfg.wht_block
    s = R.signs(42, 1, d).astype(np.float64)
    h = scipy.linalg.block_diag(*([scipy.linalg.hadamard(blk)] * (d // blk))).astype(np.float64)
    x64 = keys.astype(np.float64)
    u64 = (x64 * s) @ h.T / (math.sqrt(blk) * np.linalg.norm(x64, axis=1, keepdims=True))
    seen = set()
    for row, i, k, off in cases:
        m = m32[k]
        target = m if off == 0 else np.nextafter(m, np.float32(np.inf if off > 0 else -np.inf))
        assert u[row, i] == target
        assert abs(u64[row, i] - float(target)) <= 1e-5 * max(abs(float(m)), 1e-3)
        assert idx[row, i] == (k + 1 if off > 0 else k), (row, i, k, off)
        seen.add((k, off))
    # every midpoint is tied from both sides (the zero midpoint only exactly)
    nz = [k for k in range(len(m32)) if m32[k] != 0]
    assert seen == {(k, o) for k in nz for o in (-1, 0, 1)} | {(k, 0) for k in range(len(m32)) if m32[k] == 0}


def test_zero_key_vector():
    cfg = _cfg(128, 3)
    x = np.zeros((2, 128), np.float32)
    idx, norm16 = X.encode_keys_mse(x, cfg, 0)
    assert (norm16 == 0).all()
    c32, m32 = LM.tables_f32(128, 3)
    # u == 0 sits on the middle midpoint (0) and takes the lower index
    assert (idx == 3).all()
    khat, _ = X.dequant_f32(X.encode_slots(x, x, cfg, 0), cfg, 0)
    assert (khat == 0).all()


def _slot_hex(k_row, v_row, d, kb, vb):
    cfg = _cfg(d, kb, vb)
    return X.encode_slots(np.asarray([k_row], np.float32), np.asarray([v_row], np.float32), cfg, 0)[0]


def test_non_finite_keys_hand_worked_bytes():
    """Keys holding a NaN or an infinity, bytes worked out by hand.

    A NaN key makes the norm NaN, so 1/p and every rotated coordinate u are
    NaN; an infinite key makes the norm infinite, 1/p = 0, and every rotated
    coordinate of its Hadamard block +-inf, so u = +-inf * 0 = NaN. A NaN lies
    above no midpoint: index 0 (the count of midpoints strictly below u). The
    norm field is the fp16 of the norm: 0x7e00 (quiet NaN) or 0x7c00 (+inf).
    With D = 96 the rotation is three blocks of 32, and an infinity in block
    0 leaves blocks 1 and 2 finite: there u = z * 0 = +-0, which is above the
    midpoints below 0 only (the middle midpoint is exactly 0), index
    2^b / 2 - 1.
    """
    rng = np.random.default_rng(17)
    base64 = rng.standard_normal(64).astype(np.float32)
    v = np.zeros(64, np.float32)
    # D = 64, 3-bit: 24 code bytes of index 0, then the norm
    k = base64.copy()
    k[5] = np.nan
    assert _slot_hex(k, v, 64, 3, 4)[:26].tobytes().hex() == "00" * 24 + "007e"
    k = base64.copy()
    k[7] = np.inf
    assert _slot_hex(k, v, 64, 3, 4)[:26].tobytes().hex() == "00" * 24 + "007c"
    k = base64.copy()
    k[3] = -np.inf                          # the norm is +inf either way
    assert _slot_hex(k, v, 64, 3, 4)[:26].tobytes().hex() == "00" * 24 + "007c"
    # D = 96, infinity at element 7 (block 0)
    base96 = rng.standard_normal(96).astype(np.float32)
    v96 = np.zeros(96, np.float32)
    k = base96.copy()
    k[7] = np.inf
    # 3-bit: elements 0..31 index 0 (12 bytes); 32..95 index 3 = 0b011, eight
    # elements per 24 bits: sum_j 3 << 3j = 0x6db6db, little-endian db b6 6d
    assert _slot_hex(k, v96, 96, 3, 4)[:38].tobytes().hex() == "00" * 12 + "dbb66d" * 8 + "007c"
    # 4-bit: index 7 in two nibbles per byte
    assert _slot_hex(k, v96, 96, 4, 4)[:50].tobytes().hex() == "00" * 16 + "77" * 32 + "007c"


def test_non_finite_values_hand_worked_bytes():
    """Values holding a NaN or an infinity, bytes worked out by hand.

    min and max skip a NaN element, quiet or signalling, so the integer ramp
    0..15 with one NaN keeps scale 1 and zero 0 (fp16 0x3c00, 0x0000), and the
    NaN element takes code 0. An infinity makes the scale infinite (0x7c00) and 1/scale' = 0, so
    every code is 0 (finite elements: rint(+-0); the infinite one: inf * 0 =
    NaN -> 0); -inf is also the zero point (0xfc00).
    """
    k = np.ones(64, np.float32)
    ramp = (np.arange(64) % 16).astype(np.float32)
    off = 26                                 # value field after the 3-bit key field at D = 64
    v = ramp.copy()
    v[5] = np.nan
    # codes 0..15 pack as 10 32 54 76 98 ba dc fe; code 5 -> 0 makes byte 2 0x04
    want = "1032047698badcfe" + "1032547698badcfe" * 3 + "003c" + "0000"
    assert _slot_hex(k, v, 64, 3, 4)[off:off + 36].tobytes().hex() == want
    # a signalling NaN (quiet bit clear) is skipped the same way
    v = ramp.copy()
    v.view(np.uint32)[5] = 0x7F800001
    assert _slot_hex(k, v, 64, 3, 4)[off:off + 36].tobytes().hex() == want
    v = ramp.copy()
    v[1] = np.inf
    assert _slot_hex(k, v, 64, 3, 4)[off:off + 36].tobytes().hex() == "00" * 32 + "007c" + "0000"
    v = ramp.copy()
    v[0] = -np.inf
    assert _slot_hex(k, v, 64, 3, 4)[off:off + 36].tobytes().hex() == "00" * 32 + "007c" + "00fc"


def test_norm_correction_changes_no_bytes():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((64, 128)).astype(np.float32)
    v = rng.standard_normal((64, 128)).astype(np.float32)
    a = X.encode_slots(k, v, _cfg(128, 4, 4, nc=False), 1)
    b = X.encode_slots(k, v, _cfg(128, 4, 4, nc=True), 1)
    assert np.array_equal(a, b)
    ka, _ = X.dequant_f64(a, _cfg(128, 4, 4, nc=False), 1)
    kb_, _ = X.dequant_f64(b, _cfg(128, 4, 4, nc=True), 1)
    assert not np.allclose(ka, kb_)


def test_norm_correction_rescales_centroid_vector():
    """Under NC the dequantized key's norm equals the stored vec_norm."""
    cfg = _cfg(128, 3, 3, nc=True)
    rng = np.random.default_rng(6)
    k = rng.standard_normal((100, 128)).astype(np.float32)
    slots = X.encode_slots(k, k, cfg, 0)
    khat, _ = X.dequant_f64(slots, cfg, 0)
    n16 = X.f16_bits_to_f32(X.decode_slot_fields(slots, cfg)["norm16"])
    assert np.allclose(np.linalg.norm(khat, axis=1), n16, rtol=1e-12)


def test_fp8_slot_layout():
    cfg = C.from_cache_dtype("turboquant_k8v4", 128)
    rng = np.random.default_rng(7)
    k = rng.standard_normal((10, 128)).astype(np.float32)
    v = rng.standard_normal((10, 128)).astype(np.float32)
    slots = X.encode_slots(k, v, cfg, 0)
    assert slots.shape == (10, 196)
    assert np.array_equal(slots[:, :128], X.fp8_e4m3fn_encode(k))
    codes, s16, z16 = X.encode_values(v, 4)
    assert np.array_equal(slots[:, 128:192], X.pack_bits(codes, 4))
    assert np.array_equal(slots[:, 192] | (slots[:, 193].astype(np.uint16) << 8), s16)
    assert np.array_equal(slots[:, 194] | (slots[:, 195].astype(np.uint16) << 8), z16)


def test_two_bit_value_slot_layout():
    cfg = C.TQConfig(head_dim=128, key_quant_bits=3, value_quant_bits=2, norm_correction=True)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((10, 128)).astype(np.float32)
    v = rng.standard_normal((10, 128)).astype(np.float32)
    slots = X.encode_slots(k, v, cfg, 2)
    assert slots.shape == (10, 86)
    idx, norm16 = X.encode_keys_mse(k, cfg, 2)
    assert np.array_equal(slots[:, :48], X.pack_bits(idx, 3))
    codes, s16, z16 = X.encode_values(v, 2)
    assert codes.max() <= 3
    assert np.array_equal(slots[:, 50:82], X.pack_bits(codes, 2))
    assert np.array_equal(slots[:, 82] | (slots[:, 83].astype(np.uint16) << 8), s16)
    assert np.array_equal(slots[:, 84] | (slots[:, 85].astype(np.uint16) << 8), z16)


@pytest.mark.parametrize("preset,d", [("turboquant_4bit_nc", 128), ("turboquant_3bit_nc", 128),
                                      ("turboquant_k3v4_nc", 96), ("turboquant_k8v4", 128)])
def test_dequant_f32_close_to_exact(preset, d):
    cfg = C.from_cache_dtype(preset, d)
    rng = np.random.default_rng(8)
    k = rng.standard_normal((50, d)).astype(np.float32)
    v = rng.standard_normal((50, d)).astype(np.float32)
    slots = X.encode_slots(k, v, cfg, 2)
    k32, v32 = X.dequant_f32(slots, cfg, 2)
    k64, v64 = X.dequant_f64(slots, cfg, 2)
    assert np.allclose(k32, k64, rtol=1e-5, atol=1e-6)
    assert np.allclose(v32, v64, rtol=1e-6, atol=1e-6)


def test_pool_addressing_and_skip():
    cfg = _cfg(64, 3)
    pool = np.zeros((4, 2, 16, cfg.slot_size_aligned), np.uint8)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((5, 2, 64)).astype(np.float32)
    v = rng.standard_normal((5, 2, 64)).astype(np.float32)
    mapping = np.array([17, -1, 0, 63, 40])
    X.append(pool, k, v, mapping, cfg, 0)
    for t, sl in enumerate(mapping):
        if sl < 0:
            continue
        for h in range(2):
            want = X.encode_slots(k[t, h][None], v[t, h][None], cfg, 0)[0]
            assert np.array_equal(pool[sl // 16, h, sl % 16], want)
    written = {(s // 16, s % 16) for s in mapping if s >= 0}
    for blk in range(4):
        for off in range(16):
            if (blk, off) not in written:
                assert (pool[blk, :, off] == 0).all()
    ids = X.logical_slot_ids(np.array([2, 0, 3]), 40, 16)
    assert list(ids[:3]) == [32, 33, 34] and ids[16] == 0 and ids[39] == 3 * 16 + 7
