"""Slot encode, paged-pool addressing and dequantization (oracle; test only).

Sources:

* vLLM API page "vllm.model_executor.layers.quantization.turboquant",
  ``TurboQuantConfig``: the docstring (PolarQuant keys = Walsh-Hadamard
  rotation + Lloyd-Max scalar quantization; uniform quantization for values;
  FP8 keys when key_quant_bits is 8; norm correction re-normalizes the
  centroid vector to unit norm before the inverse rotation at dequant) and
  the byte layouts in ``key_packed_size`` (MSE indices then an fp16 vec_norm,
  or D FP8 bytes), ``value_packed_size`` (codes then fp16 scale and fp16
  zero) and ``slot_size`` ([key_packed | value_packed] per head per
  position, rounded up to an even size by ``slot_size_aligned``).
* prhub summary of vLLM PR #39931, source snippet from ``interface.py``: a
  TurboQuant page holds ``block_size * num_kv_heads * slot_size_aligned``
  bytes; the order inside a page is not fixed there.

Readings taken where the pages are silent (all also listed in the design doc):

* What is quantized: the rotated unit vector Pi x / ||x||; the norm is stored
  separately as fp16, and norm correction changes only dequant and decode
  (packed bytes are identical with it on or off).
* Key fp32 op order: squares, then a pairwise tree with adjacent pairing
  inside each Hadamard block, block totals added left to right; correctly
  rounded sqrt; fp16 by round-to-nearest-even; signs applied; butterflies
  ascending; p = n * fp32(sqrt(B)); r = 1/p (0 when n == 0); u = z * r.
* Index: number of fp32 midpoints strictly below u (ties go to the lower
  index).
* Bit packing: LSB-first bitstream, element j at bits [j*b, (j+1)*b); fields
  in the listed order; fp16 fields little-endian; pad bits and pad byte 0.
* FP8 keys: OCP E4M3FN (bias 7, max 448), round-to-nearest-even, values
  beyond the range saturate to +-448, the sign of zero is kept, NaN -> 0x7f
  with its sign. Unscaled.
* Values: asymmetric min/max per (token, head) vector. scale = (max - min)/L
  in fp32, L = 2**bits - 1; scale and zero (= min) stored as fp16; codes are
  clamp(rint((v - zero') * (1/scale')), 0, L) computed from the stored
  (fp16-rounded) scale' and zero'; 1/scale' is 0 when scale' is 0; rint is
  half-to-even.
* Non-finite inputs: min and max skip NaN elements (IEEE minNum / maxNum);
  a NaN quotient takes code 0; a key coordinate whose rotated value is NaN
  (a NaN or infinite key makes 1/p zero or NaN) is above no midpoint and
  gets index 0; fp16 fields of NaN or infinite quantities are the IEEE
  conversions of those values.
* Pool layout: [num_blocks][num_kv_heads][block_size][slot_size_aligned]
  bytes; token t goes to block slot_mapping[t] // block_size at offset
  slot_mapping[t] % block_size; slot_mapping -1 means skip.
* Dequant in fp32 (the exact target of the library's dequant): centroids
  looked up in the fp32 table; with norm correction divided by their norm
  (same tree, correctly rounded sqrt, then multiplied by the fp32 reciprocal);
  butterflies ascending; multiplied by fp32(n16 * fp32(1/sqrt(B))); signs
  applied. Values: fp32(fp32(scale' * code) + zero'), no fused multiply-add.
"""

from __future__ import annotations

import math

import numpy as np

from . import lloyd_max, rotation
from .config import TQConfig

# ----------------------------------------------------------------------------
# scalar formats


def f32_to_f16_bits(x) -> np.ndarray:
    """fp32 -> IEEE binary16 bits, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_value(code: int) -> float:
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        return m * 2.0 ** -9
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Non-negative finite E4M3FN values, codes 0x00..0x7e, ascending.
E4M3_VALUES = np.array([_e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
E4M3_MAX = 448.0


def fp8_e4m3fn_encode(x) -> np.ndarray:
    """Nearest E4M3FN code by its plain definition (see module header)."""
    x = np.asarray(x, dtype=np.float32)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.minimum(np.abs(x.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(E4M3_VALUES, a, side="left")  # E[hi-1] < a <= E[hi]
    hi = np.clip(hi, 0, len(E4M3_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - E4M3_VALUES[lo]
    d_hi = E4M3_VALUES[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a == E4M3_VALUES[hi], hi, pick)
    code = pick.astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def fp8_e4m3fn_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E4M3_VALUES[np.minimum(code & 0x7F, 0x7E)]
    val = np.where((code & 0x80) != 0, -mag, mag)
    val = np.where((code & 0x7F) == 0x7F, np.nan, val)
    return val.astype(np.float32)


# ----------------------------------------------------------------------------
# bit packing


def pack_bits(codes, bits: int) -> np.ndarray:
    """[N, D] codes -> [N, ceil(D*bits/8)] bytes, LSB-first bitstream."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, d = codes.shape
    planes = ((codes[:, :, None] >> np.arange(bits, dtype=np.uint32)) & 1).astype(np.uint8)
    stream = planes.reshape(n, d * bits)
    nbytes = math.ceil(d * bits / 8)
    pad = nbytes * 8 - d * bits
    if pad:
        stream = np.concatenate([stream, np.zeros((n, pad), np.uint8)], axis=1)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack_bits(packed, bits: int, d: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    stream = np.unpackbits(packed, axis=1, bitorder="little")[:, : d * bits]
    planes = stream.reshape(n, d, bits).astype(np.uint32)
    return (planes << np.arange(bits, dtype=np.uint32)).sum(axis=2).astype(np.uint8)


def _le16(bits16) -> np.ndarray:
    b = np.asarray(bits16, dtype=np.uint16)
    return np.stack([(b & 0xFF).astype(np.uint8), (b >> 8).astype(np.uint8)], axis=-1)


# ----------------------------------------------------------------------------
# key encode


def sumsq_tree_f32(x: np.ndarray, block: int) -> np.ndarray:
    """sum_j x_j^2 in fp32: adjacent-pair tree inside each block, block totals
    added left to right."""
    a = np.asarray(x, dtype=np.float32)
    a = a * a
    n, d = a.shape
    a = a.reshape(n, d // block, block)
    while a.shape[-1] > 1:
        a = a[..., 0::2] + a[..., 1::2]
    totals = a[..., 0]
    acc = totals[:, 0]
    for k in range(1, totals.shape[1]):
        acc = acc + totals[:, k]
    return acc.astype(np.float32)


def encode_keys_mse(x, cfg: TQConfig, layer_idx: int):
    """Keys [N, D] (fp32 values) -> (indices [N, D] uint8, vec_norm fp16 bits [N])."""
    x = np.asarray(x, dtype=np.float32)
    block = cfg.wht_block
    s = rotation.signs(cfg.seed, layer_idx, cfg.head_dim)
    _, m32 = lloyd_max.tables_f32(cfg.head_dim, cfg.key_mse_bits)
    # (non-finite keys: the steps below run unchanged; see the header)
    with np.errstate(invalid="ignore", over="ignore"):
        n = np.sqrt(sumsq_tree_f32(x, block)).astype(np.float32)
        norm16 = f32_to_f16_bits(n)
        z = rotation.butterfly_f32(x * s, block)
        p = n * np.float32(math.sqrt(block))
        with np.errstate(divide="ignore"):
            r = np.where(n == 0, np.float32(0), np.float32(1) / p).astype(np.float32)
        u = z * r[:, None]
    # index = number of midpoints strictly below u, counted as written: a NaN
    # coordinate (from a NaN or infinite key) is below none and gets 0
    idx = (u[:, :, None] > m32[None, None, :]).sum(axis=2).astype(np.uint8)
    return idx, norm16


def encode_keys_fp8(x) -> np.ndarray:
    return fp8_e4m3fn_encode(np.asarray(x, dtype=np.float32))


# ----------------------------------------------------------------------------
# value encode


def encode_values(v, bits: int):
    """Values [N, D] -> (codes [N, D] uint8, scale fp16 bits [N], zero fp16 bits [N])."""
    v = np.asarray(v, dtype=np.float32)
    levels = np.float32(2 ** bits - 1)
    # minimum and maximum over the elements that are numbers (IEEE 754
    # minNum / maxNum): a NaN element does not make the scale NaN
    with np.errstate(invalid="ignore"):
        mn = np.fmin.reduce(v, axis=1)
        mx = np.fmax.reduce(v, axis=1)
    scale32 = (mx - mn) / levels
    s16 = f32_to_f16_bits(scale32)
    z16 = f32_to_f16_bits(mn)
    s1 = f16_bits_to_f32(s16)
    z1 = f16_bits_to_f32(z16)
    with np.errstate(divide="ignore"):
        inv = np.where(s1 == 0, np.float32(0), np.float32(1) / s1).astype(np.float32)
    with np.errstate(invalid="ignore"):
        q = np.rint((v - z1[:, None]) * inv[:, None])
    # a NaN quotient (NaN element, or an infinite one times 1/inf = 0) takes
    # the lowest code
    q = np.where(np.isnan(q), np.float32(0), q)
    codes = np.clip(q, 0, levels).astype(np.uint8)
    return codes, s16, z16


# ----------------------------------------------------------------------------
# slots


def encode_slots(k, v, cfg: TQConfig, layer_idx: int) -> np.ndarray:
    """K, V [N, D] (fp32 values) -> slots [N, slot_size_aligned] uint8."""
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    n = k.shape[0]
    if cfg.key_fp8:
        key_field = encode_keys_fp8(k)
    else:
        idx, norm16 = encode_keys_mse(k, cfg, layer_idx)
        key_field = np.concatenate([pack_bits(idx, cfg.key_mse_bits), _le16(norm16)], axis=1)
    codes, s16, z16 = encode_values(v, cfg.value_quant_bits)
    val_field = np.concatenate(
        [pack_bits(codes, cfg.value_quant_bits), _le16(s16), _le16(z16)], axis=1)
    slot = np.concatenate([key_field, val_field], axis=1)
    assert key_field.shape[1] == cfg.key_packed_size
    assert val_field.shape[1] == cfg.value_packed_size
    if cfg.slot_size_aligned != cfg.slot_size:
        slot = np.concatenate([slot, np.zeros((n, 1), np.uint8)], axis=1)
    return slot


def decode_slot_fields(slots, cfg: TQConfig) -> dict:
    """Split slots [N, S] into their fields (no arithmetic beyond unpacking)."""
    slots = np.asarray(slots, dtype=np.uint8)
    d = cfg.head_dim
    out = {}
    kp = cfg.key_packed_size
    if cfg.key_fp8:
        out["fp8"] = slots[:, :d]
    else:
        nb = kp - 2
        out["idx"] = unpack_bits(slots[:, :nb], cfg.key_mse_bits, d)
        out["norm16"] = slots[:, nb].astype(np.uint16) | (slots[:, nb + 1].astype(np.uint16) << 8)
    vb = cfg.value_packed_size - 4
    vfield = slots[:, kp:kp + cfg.value_packed_size]
    out["codes"] = unpack_bits(vfield[:, :vb], cfg.value_quant_bits, d)
    out["scale16"] = vfield[:, vb].astype(np.uint16) | (vfield[:, vb + 1].astype(np.uint16) << 8)
    out["zero16"] = vfield[:, vb + 2].astype(np.uint16) | (vfield[:, vb + 3].astype(np.uint16) << 8)
    return out


# ----------------------------------------------------------------------------
# paged pool


def pool_shape(cfg: TQConfig, num_blocks: int, num_kv_heads: int, block_size: int):
    return (num_blocks, num_kv_heads, block_size, cfg.slot_size_aligned)


def write_pool(pool: np.ndarray, slots: np.ndarray, slot_mapping) -> None:
    """pool [nb, H, bs, S]; slots [T, H, S]; slot_mapping [T] (-1 = skip)."""
    bs = pool.shape[2]
    for t, sl in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if sl < 0:
            continue
        pool[sl // bs, :, sl % bs, :] = slots[t]


def append(pool, k, v, slot_mapping, cfg: TQConfig, layer_idx: int) -> None:
    """Quantize-and-append: K, V [T, H, D] -> pool at slot_mapping."""
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    t, h, d = k.shape
    if t == 0:
        return
    slots = encode_slots(k.reshape(t * h, d), v.reshape(t * h, d), cfg, layer_idx)
    write_pool(pool, slots.reshape(t, h, -1), slot_mapping)


def gather_slots(pool: np.ndarray, slot_ids, head: int) -> np.ndarray:
    """Slots [n, S] of one KV head at physical slot ids."""
    bs = pool.shape[2]
    ids = np.asarray(slot_ids, dtype=np.int64)
    return pool[ids // bs, head, ids % bs, :]


def logical_slot_ids(block_table_row, length: int, block_size: int) -> np.ndarray:
    """Physical slot ids of logical positions 0..length-1 of one sequence."""
    pos = np.arange(length, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[pos // block_size]
    return blocks * block_size + pos % block_size


# ----------------------------------------------------------------------------
# dequant


def dequant_f32(slots, cfg: TQConfig, layer_idx: int):
    """Slots [N, S] -> (K_hat, V_hat) [N, D] fp32, fixed op order."""
    f = decode_slot_fields(slots, cfg)
    d = cfg.head_dim
    block = cfg.wht_block
    if cfg.key_fp8:
        k = fp8_e4m3fn_decode(f["fp8"])
    else:
        s = rotation.signs(cfg.seed, layer_idx, d)
        c32, _ = lloyd_max.tables_f32(d, cfg.key_mse_bits)
        y = c32[f["idx"]]
        if cfg.norm_correction:
            cn = np.sqrt(sumsq_tree_f32(y, block)).astype(np.float32)
            y = y * (np.float32(1) / cn)[:, None]
        w = rotation.butterfly_f32(y, block)
        rb = np.float32(1.0 / math.sqrt(block))
        fac = f16_bits_to_f32(f["norm16"]) * rb
        k = s * (w * fac[:, None])
    s1 = f16_bits_to_f32(f["scale16"])
    z1 = f16_bits_to_f32(f["zero16"])
    vv = (s1[:, None] * f["codes"].astype(np.float32)) + z1[:, None]
    return k.astype(np.float32), vv.astype(np.float32)


def dequant_f64(slots, cfg: TQConfig, layer_idx: int):
    """Slots [N, S] -> (K_hat, V_hat) [N, D] float64: the exact values the
    stored fields describe (the dequantized cache of the plain definition)."""
    f = decode_slot_fields(slots, cfg)
    d = cfg.head_dim
    block = cfg.wht_block
    if cfg.key_fp8:
        k = fp8_e4m3fn_decode(f["fp8"]).astype(np.float64)
    else:
        s = rotation.signs(cfg.seed, layer_idx, d)
        c32, _ = lloyd_max.tables_f32(d, cfg.key_mse_bits)
        y = c32[f["idx"]].astype(np.float64)
        if cfg.norm_correction:
            y = y / np.linalg.norm(y, axis=1, keepdims=True)
        n16 = f16_bits_to_f32(f["norm16"]).astype(np.float64)
        k = rotation.unrotate_f64(y, s, block) * n16[:, None]
    s1 = f16_bits_to_f32(f["scale16"]).astype(np.float64)
    z1 = f16_bits_to_f32(f["zero16"]).astype(np.float64)
    vv = s1[:, None] * f["codes"].astype(np.float64) + z1[:, None]
    return k, vv
