"""Decode attention over the compressed cache (oracle; test only).

Plain definition (float64): for sequence b and query head g, with KV head
h = g // (Hq / Hkv), the attended tokens are the sequence's compressed
positions 0..len_b-1, read through its block table and dequantized, followed
by the sequence's exact ring-buffer tokens. Scores are scale * (q . k), the
output is the softmax-weighted sum of the values.

Sources:

* hnwysp.cn article on the stand-alone ``turboquant`` project, section on
  the next directions, direction 1 (the fused decode kernel): one pass over
  the compressed data, a flash-attention style online softmax advanced block
  by block, no materialised FP16 KV, and the query rotated forward (q Pi^T)
  instead of rotating keys back.
* Same article, section on the write path (ring buffer + lazy merge): recent
  decode tokens sit in a 128-token bf16 exact ring buffer, compressed as a
  whole chunk when it overflows.
* vLLM API page, ``TurboQuantConfig`` docstring: norm correction
  re-normalizes the centroid vector before the inverse rotation.

Readings: softmax scale 1/sqrt(D) unless given; GQA maps query head g to KV
head g // G; ring tokens are exact bf16 keys/values attended with the raw
(unrotated) query; a sequence with no tokens outputs zeros; the output is
float64 here and fp32 in the library.

Continuation prefill (``prefill_attention``): the API page keeps the
centroid table even for FP8 keys because continuation prefill dequantizes
the cache (``mse_bits`` docstring). Reading: a new chunk of C tokens of a
sequence with L compressed tokens attends, token t of the chunk, to the L
dequantized history tokens and to the chunk's own exact tokens 0..t
(causal), with the same scale and GQA mapping as decode.

``rotated_scores`` computes the fused kernel's form
n16 * <Pi q, c> (c re-normalized under norm correction) and
``tests/test_oracle_attention.py`` checks it equals q . k_hat to 1e-12.
"""

from __future__ import annotations

import math

import numpy as np

from . import codec, lloyd_max, rotation
from .config import TQConfig


def softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """q [G, D], k [T, D], v [T, D] (float64) -> [G, D]; zeros when T == 0."""
    g, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((g, d), dtype=np.float64)
    s = scale * (q @ k.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def sequence_kv(pool, block_table_row, length: int, head: int, cfg: TQConfig,
                layer_idx: int):
    """Dequantized (float64) K, V of one sequence and KV head."""
    bs = pool.shape[2]
    ids = codec.logical_slot_ids(block_table_row, length, bs)
    slots = codec.gather_slots(pool, ids, head)
    return codec.dequant_f64(slots, cfg, layer_idx)


def decode_attention(q, pool, block_tables, seq_lens, cfg: TQConfig, layer_idx: int,
                     ring_k=None, ring_v=None, ring_lens=None, scale=None) -> np.ndarray:
    """q [B, Hq, D] -> out [B, Hq, D] float64.

    pool [num_blocks, Hkv, block_size, S] uint8; block_tables [B, max_blocks];
    seq_lens [B]; ring_k / ring_v [B, Hkv, ring_cap, D] (float values of the
    bf16 ring) and ring_lens [B], or None.
    """
    q = np.asarray(q, dtype=np.float64)
    b_s, hq, d = q.shape
    hkv = pool.shape[1]
    grp = hq // hkv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((b_s, hq, d), dtype=np.float64)
    for b in range(b_s):
        for h in range(hkv):
            k, v = sequence_kv(pool, block_tables[b], int(seq_lens[b]), h, cfg, layer_idx)
            if ring_k is not None and ring_lens is not None and int(ring_lens[b]) > 0:
                r = int(ring_lens[b])
                k = np.concatenate([k, np.asarray(ring_k[b, h, :r], np.float64)], axis=0)
                v = np.concatenate([v, np.asarray(ring_v[b, h, :r], np.float64)], axis=0)
            out[b, h * grp:(h + 1) * grp] = softmax_attend(q[b, h * grp:(h + 1) * grp], k, v, scale)
    return out


def rotated_scores(q_row, slots, cfg: TQConfig, layer_idx: int) -> np.ndarray:
    """q . k_hat for MSE keys computed in the rotated basis, float64:
    n16 * <Pi q, c_idx> (c_idx / ||c_idx|| under norm correction)."""
    assert not cfg.key_fp8
    f = codec.decode_slot_fields(slots, cfg)
    s = rotation.signs(cfg.seed, layer_idx, cfg.head_dim)
    q_rot = rotation.rotate_f64(np.asarray(q_row, np.float64), s, cfg.wht_block)
    c32, _ = lloyd_max.tables_f32(cfg.head_dim, cfg.key_mse_bits)
    y = c32[f["idx"]].astype(np.float64)
    dots = y @ q_rot
    if cfg.norm_correction:
        dots = dots / np.linalg.norm(y, axis=1)
    return codec.f16_bits_to_f32(f["norm16"]).astype(np.float64) * dots


def prefill_attention(q, k_chunk, v_chunk, cu_chunk, pool, block_tables, hist_lens, cfg: TQConfig,
                      layer_idx: int, scale=None) -> np.ndarray:
    """q [N, Hq, D], k_chunk / v_chunk [N, Hkv, D] (float values of the exact
    chunk tokens), cu_chunk [B + 1] (sequence b's chunk is rows
    cu_chunk[b]..cu_chunk[b+1]-1), hist_lens [B] -> out [N, Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    n, hq, d = q.shape
    hkv = pool.shape[1]
    grp = hq // hkv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, hq, d), dtype=np.float64)
    for b in range(len(cu_chunk) - 1):
        r0, r1 = int(cu_chunk[b]), int(cu_chunk[b + 1])
        for h in range(hkv):
            kh, vh = sequence_kv(pool, block_tables[b], int(hist_lens[b]), h, cfg, layer_idx)
            kc = np.asarray(k_chunk[r0:r1, h], np.float64)
            vc = np.asarray(v_chunk[r0:r1, h], np.float64)
            for t in range(r1 - r0):
                k = np.concatenate([kh, kc[:t + 1]], axis=0)
                v = np.concatenate([vh, vc[:t + 1]], axis=0)
                out[r0 + t, h * grp:(h + 1) * grp] = softmax_attend(q[r0 + t, h * grp:(h + 1) * grp], k, v, scale)
    return out
