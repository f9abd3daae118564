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
