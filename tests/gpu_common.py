"""Shared helpers for the GPU parity tests (not a test module)."""

from __future__ import annotations

import sys

import numpy as np

from oracle import codec as OX
from oracle import config as OC

# Relative L2 tolerance on attention outputs (the target's stated bound).
ATTN_RTOL = 2e-3


def announce(msg: str) -> None:
    """Print what the next GPU step is, flushed, so a crash names its case."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def oracle_cfg(cfg) -> OC.TQConfig:
    """The oracle's config with the same fields as a library Config."""
    return OC.TQConfig(head_dim=cfg.head_dim, key_quant_bits=cfg.key_quant_bits,
                       value_quant_bits=cfg.value_quant_bits, seed=int(cfg.seed),
                       norm_correction=bool(cfg.norm_correction))


def oracle_pool(ocfg, layer, k, v, slot_mapping, num_blocks, hkv, block_size):
    pool = np.zeros((num_blocks, hkv, block_size, ocfg.slot_size_aligned), np.uint8)
    OX.append(pool, k, v, slot_mapping, ocfg, layer)
    return pool


def rel_l2(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    if den == 0:
        return float(np.linalg.norm(got))
    return float(np.linalg.norm(got - want) / den)


def per_head_rel_l2(got, want):
    """Max over (sequence, query head) of the relative L2 error; exact zeros
    where the reference is zero."""
    worst = 0.0
    b_s, hq, _ = want.shape
    for b in range(b_s):
        for h in range(hq):
            w = want[b, h]
            g = got[b, h]
            if not np.any(w):
                assert not np.any(g), f"expected zeros at ({b},{h})"
                continue
            worst = max(worst, rel_l2(g, w))
    return worst


def as_f32_host(t) -> np.ndarray:
    return t.float().cpu().numpy()


def attention_conditioning(q, pool, tables, lens, ocfg, layer, ring_k=None, ring_v=None, ring_lens=None):
    """Per (sequence, query head): the condition number of the softmax-
    weighted value sum with respect to the terms the decode kernel adds, and
    the number of attended tokens n.

    The kernel carries a compressed token's value v_t = s'_t c_t + z'_t as
    two fp32 terms: the centred codes c_t - c0 (c0 = 2^(b-1)) times the
    weight p_t s'_t, and z'_t + c0 s'_t times p_t; a ring token's bf16 value
    is one term. A relative perturbation e of every term (its weight, or its
    share of an fp32 sum) moves the output by at most kappa * e relative to
    its norm, with

        kappa = sum_t p_t m_t / |sum_t p_t v_t|,
        m_t = |s'_t| |c_t - c0| + sqrt(D) |z'_t + c0 s'_t|   (compressed),
        m_t = |v_t|                                          (ring),

    float64, from the oracle's decoding of the stored fields."""
    import math
    from oracle import attention as OA
    q = np.asarray(q, np.float64)
    b_s, hq, d = q.shape
    hkv = pool.shape[1]
    g = hq // hkv
    bs = pool.shape[2]
    kap = np.zeros((b_s, hq))
    n_tok = np.zeros(b_s, np.int64)
    for b in range(b_s):
        for h in range(hkv):
            k, v = OA.sequence_kv(pool, tables[b], int(lens[b]), h, ocfg, layer)
            f = OX.decode_slot_fields(OX.gather_slots(pool, OX.logical_slot_ids(tables[b], int(lens[b]), bs), h), ocfg)
            s1 = OX.f16_bits_to_f32(f["scale16"]).astype(np.float64)
            z1 = OX.f16_bits_to_f32(f["zero16"]).astype(np.float64)
            c0 = float(1 << (ocfg.value_quant_bits - 1))
            cc = f["codes"].astype(np.float64) - c0
            mag = np.abs(s1) * np.linalg.norm(cc, axis=1) + math.sqrt(d) * np.abs(z1 + c0 * s1)
            if ring_lens is not None and int(ring_lens[b]) > 0:
                r = int(ring_lens[b])
                rv = np.asarray(ring_v[b, h, :r], np.float64)
                k = np.concatenate([k, np.asarray(ring_k[b, h, :r], np.float64)])
                v = np.concatenate([v, rv])
                mag = np.concatenate([mag, np.linalg.norm(rv, axis=1)])
            n_tok[b] = k.shape[0]
            if k.shape[0] == 0:
                continue
            s = (q[b, h * g:(h + 1) * g] @ k.T) / math.sqrt(d)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v
            kap[b, h * g:(h + 1) * g] = (p @ mag) / np.linalg.norm(o, axis=1)
    return kap, n_tok
