"""Cache-management rules around the hot path (oracle; test infrastructure only).

Sources:
- vLLM API page "vllm.model_executor.layers.quantization.turboquant",
  ``TurboQuantConfig.get_boundary_skip_layers``: the first and last n layers
  (n = 2 by default) keep the unquantized cache, n is capped at half the
  layer count, indices are deduplicated, sorted and returned as strings; n <= 0
  or no layers gives an empty list.
- prhub summary of vLLM PR #39931 (implementation breakdown item 1 and the
  interface.py snippet): hybrid models get an empty skip list; the per-token
  attention page is the TurboQuant page (block size 1, ``tq_slot_size`` =
  slot_size_aligned per KV head), and when skip layers exist it is the least
  common multiple of that and the unquantized page of a skip layer, not the
  maximum.
- hnwysp.cn article on the stand-alone turboquant project, write-path section:
  decode tokens enter a 128-token bf16 exact ring buffer, which is compressed
  as one whole chunk when it overflows.

Readings (the pages leave these open):
- The unquantized skip-layer page at block size 1 holds K and V of every KV
  head: 2 * num_kv_heads * head_dim * dtype_bytes (the usual full-attention
  page; the snippet names the spec but not its formula).
- Overflow means a new token arriving at a full ring: a decode step first
  flushes full rings (their tokens become compressed positions
  seq_len .. seq_len + cap - 1 in order, the ring empties), then appends the
  new token. So between steps a ring holds 0..cap tokens, and a full ring is
  attended exactly until the next token arrives.

Pins: hand-worked skip lists and page sizes; the ring's end state against a
direct append of the same tokens (tests/test_oracle_cache.py).
"""

from __future__ import annotations

import math

import numpy as np

from oracle import codec as OX
from oracle.config import TQConfig


def boundary_skip_layers(num_layers: int, n: int = 2, hybrid: bool = False) -> list[str]:
    """Layers that keep the unquantized cache: first and last n of a dense model."""
    if hybrid or n <= 0 or num_layers <= 0:
        return []
    n = min(n, num_layers // 2)
    keep = set(range(n)) | set(range(num_layers - n, num_layers))
    return [str(i) for i in sorted(keep)]


def tq_page_bytes_1_token(cfg: TQConfig, num_kv_heads: int) -> int:
    """TurboQuant attention page at block size 1: one aligned slot per KV head."""
    return num_kv_heads * cfg.slot_size_aligned


def skip_page_bytes_1_token(head_dim: int, num_kv_heads: int, dtype_bytes: int) -> int:
    """Unquantized skip-layer page at block size 1: K and V rows of every head."""
    return 2 * num_kv_heads * head_dim * dtype_bytes


def attn_page_bytes_1_token(cfg: TQConfig, num_kv_heads: int, skip_dtype_bytes: int = 0) -> int:
    """Per-token page every attention layer shares: the TurboQuant page, or its
    lcm with the skip-layer page when skip layers exist (skip_dtype_bytes > 0)."""
    tq = tq_page_bytes_1_token(cfg, num_kv_heads)
    if skip_dtype_bytes <= 0:
        return tq
    return math.lcm(tq, skip_page_bytes_1_token(cfg.head_dim, num_kv_heads, skip_dtype_bytes))


class RingState:
    """Per-sequence compressed history (paged pool) plus the exact ring.

    pool: uint8 [num_blocks][Hkv][block_size][S]; tables: int32 [B][max_blocks];
    seq_lens: compressed tokens per sequence; ring_k / ring_v: float32 values
    of bf16 tokens [B][Hkv][cap][D]; ring_lens: ring tokens per sequence.
    """

    def __init__(self, cfg: TQConfig, layer: int, pool, tables, seq_lens, ring_k, ring_v, ring_lens):
        self.cfg, self.layer = cfg, layer
        self.pool, self.tables = pool, np.asarray(tables)
        self.seq_lens = np.array(seq_lens, dtype=np.int64)
        self.ring_k, self.ring_v = ring_k, ring_v
        self.ring_lens = np.array(ring_lens, dtype=np.int64)
        self.cap = ring_k.shape[2]

    def flush_full(self) -> None:
        """Compress every full ring as one chunk at the sequence's next positions."""
        bs = self.pool.shape[2]
        for b in np.nonzero(self.ring_lens >= self.cap)[0]:
            pos = self.seq_lens[b] + np.arange(self.cap)
            slots = self.tables[b, pos // bs].astype(np.int64) * bs + pos % bs
            k = np.transpose(self.ring_k[b], (1, 0, 2))  # [cap, Hkv, D]
            v = np.transpose(self.ring_v[b], (1, 0, 2))
            OX.append(self.pool, k, v, slots, self.cfg, self.layer)
            self.seq_lens[b] += self.cap
            self.ring_lens[b] = 0

    def append(self, k_new, v_new) -> None:
        """Each sequence's new token (k_new, v_new [B][Hkv][D]) at its ring's end."""
        for b in range(len(self.ring_lens)):
            r = self.ring_lens[b]
            if r < self.cap:
                self.ring_k[b, :, r] = k_new[b]
                self.ring_v[b, :, r] = v_new[b]
                self.ring_lens[b] = r + 1

    def step(self, k_new, v_new) -> None:
        """One decode step's write: flush rings that are full, then append."""
        self.flush_full()
        self.append(k_new, v_new)
