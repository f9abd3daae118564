"""Builds a workload's resident GPU state: generated K/V appended through the
library's quantize-append into a paged pool, block tables, lengths, queries
and the ring. Orchestration only (random data and calls into the library);
no arithmetic of the method lives here.
"""

from __future__ import annotations

import math

import numpy as np

from . import KVSource, Workload, block_tables, sequence_lengths, slot_ids_for


class Built:
    """Resident state of one workload on the GPU."""

    def __init__(self):
        self.pools = []
        self.captured = {}


def build(w: Workload, device="cuda", n_pools: int = 1, capture=(), fill_chunk: int = 65536,
          extra_blocks: int = 0):
    """Fill ``n_pools`` independent pools with the workload's compressed tokens.

    capture: sequence indices whose generated K/V (pool 0) are kept on the
    host as float32 arrays [len, Hkv, D] for oracle checks.
    """
    import torch

    import compressed_decode_attention_quantize_amd as tq

    cfg = tq.config_from_preset(w.preset, w.head_dim) if w.preset else \
        tq.config_init(w.head_dim, w.key_bits, w.value_bits, w.norm_correction, 42)
    lens = sequence_lengths(w)
    tables, num_blocks, spare = block_tables(w, lens, extra_blocks)
    S = cfg.slot_size_aligned
    out = Built()
    out.w = w
    out.cfg = cfg
    out.lens_np = lens
    out.tables_np = tables
    out.num_blocks = num_blocks
    out.spare_blocks = spare
    out.tables = torch.from_numpy(tables).to(device)
    out.seq_lens = torch.from_numpy(lens.astype(np.int32)).to(device)
    out.max_seq_len = int(lens.max()) if len(lens) else 0
    capture = set(capture)
    for pi in range(n_pools):
        pool = torch.zeros((num_blocks, w.num_kv_heads, w.block_size, S), dtype=torch.uint8, device=device)
        src = KVSource(w, device, stream_id=pi)
        for b in range(w.batch):
            n = int(lens[b])
            keep_k, keep_v = [], []
            for start in range(0, n, fill_chunk):
                cnt = min(fill_chunk, n - start)
                k, v = src.kv(cnt)
                ids = torch.from_numpy(slot_ids_for(tables, b, start, cnt, w.block_size)).to(device)
                tq.quantize_append(cfg, 0, k, v, ids, pool)
                if pi == 0 and b in capture:
                    keep_k.append(k.float().cpu().numpy())
                    keep_v.append(v.float().cpu().numpy())
            if pi == 0 and b in capture:
                d = w.head_dim
                out.captured[b] = (np.concatenate(keep_k) if keep_k else np.zeros((0, w.num_kv_heads, d), np.float32),
                                   np.concatenate(keep_v) if keep_v else np.zeros((0, w.num_kv_heads, d), np.float32))
        out.pools.append(pool)
        if pi == 0:
            out.q = src.q()
            if w.ring:
                out.ring_k, out.ring_v = src.ring()
                out.ring_lens = torch.full((w.batch,), w.ring, dtype=torch.int32, device=device)
            else:
                out.ring_k = out.ring_v = out.ring_lens = None
            # one new token per sequence for the decode step's append
            out.step_k, out.step_v = src.kv(w.batch)
            last = [slot_ids_for(tables, b, max(int(lens[b]) - 1, 0), 1, w.block_size)[0] if lens[b] > 0 else -1
                    for b in range(w.batch)]
            out.step_slots = torch.tensor(last, dtype=torch.int64, device=device)
    torch.cuda.synchronize()
    return out


def prefill_source(w: Workload, device="cuda"):
    """Generator of the concurrent prefill's K/V (a sequence outside the batch)."""
    return KVSource(w, device, stream_id=99)


def spare_slot_ids(built, count: int):
    """Physical slot ids of `count` tokens laid out over the spare blocks."""
    bs = built.w.block_size
    need = math.ceil(count / bs)
    blocks = np.asarray(built.spare_blocks[:need], dtype=np.int64)
    assert len(blocks) == need, "not enough spare blocks"
    pos = np.arange(count, dtype=np.int64)
    return blocks[pos // bs] * bs + pos % bs


def prepare_steps(built, split_tokens: int = 0):
    """One decode step per pool, as bench.py times it: append one new token per
    sequence (quantize-append at the sequence's last compressed position),
    then decode attention over every sequence's full context (compressed +
    ring). Returns a list of (quantize_call, decode_call) pairs sharing the
    same output and workspace."""
    import compressed_decode_attention_quantize_amd as tq

    b = built
    steps = []
    out = ws = None
    for pool in b.pools:
        qc = tq.prepare_quantize(b.cfg, 0, b.step_k, b.step_v, b.step_slots, pool)
        dc = tq.prepare_decode(b.cfg, 0, b.q, pool, b.tables, b.seq_lens, b.max_seq_len,
                               b.ring_k, b.ring_v, b.ring_lens, out=out, workspace=ws,
                               split_tokens=split_tokens)
        out, ws = dc.out, dc.workspace
        steps.append((qc, dc))
    return steps


def decode_bytes(built) -> int:
    """Algorithmic bytes one decode launch must move: every attended slot,
    the ring's bf16 K and V, the block-table entries in use, the lengths, q
    and the fp32 output. Split partials are not counted."""
    w = built.w
    s = built.cfg.slot_size_aligned
    lens = built.lens_np.astype(np.int64)
    slots = int(lens.sum()) * w.num_kv_heads * s
    ring = w.batch * w.ring * w.num_kv_heads * w.head_dim * 2 * 2
    tables = int(np.ceil(lens / w.block_size).sum()) * 4
    q_bytes = w.batch * w.num_q_heads * w.head_dim * (4 if w.in_dtype == "f32" else 2)
    out_bytes = w.batch * w.num_q_heads * w.head_dim * 4
    lens_bytes = w.batch * 4 * (2 if w.ring else 1)
    return slots + ring + tables + q_bytes + out_bytes + lens_bytes


def quantize_bytes_per_token(built) -> int:
    """Algorithmic bytes of quantize-append per token (all KV heads): K and V
    in, slots out, one int64 slot id."""
    w = built.w
    ib = 4 if w.in_dtype == "f32" else 2
    return 2 * w.num_kv_heads * w.head_dim * ib + w.num_kv_heads * built.cfg.slot_size_aligned + 8
