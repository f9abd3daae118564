"""Pins of the oracle's cache-management rules: boundary skip lists and page
sizes worked by hand from the API page and the PR summary, and the ring
buffer's end state against a direct append of the same tokens."""

import math

import numpy as np
import pytest

from oracle import cache as OC
from oracle import codec as OX
from oracle import config as C


@pytest.mark.parametrize("num_layers,n,want", [
    (32, 2, ["0", "1", "30", "31"]),
    (10, 3, ["0", "1", "2", "7", "8", "9"]),
    (4, 2, ["0", "1", "2", "3"]),
    (3, 2, ["0", "2"]),        # n capped at 3 // 2 = 1
    (2, 2, ["0", "1"]),
    (1, 2, []),                # 1 // 2 = 0 layers each side
    (5, 0, []),
    (0, 2, []),
    (7, -1, []),
])
def test_boundary_skip_layers_dense(num_layers, n, want):
    assert OC.boundary_skip_layers(num_layers, n) == want


def test_boundary_skip_layers_default_and_hybrid():
    assert OC.boundary_skip_layers(28) == ["0", "1", "26", "27"]
    assert OC.boundary_skip_layers(48, hybrid=True) == []


@pytest.mark.parametrize("preset,hkv,dtype_bytes,tq,skip,want", [
    # 8 * 134 = 1072 = 2^4 * 67; 2 * 8 * 128 * 2 = 4096 = 2^12 -> 2^12 * 67
    ("turboquant_4bit_nc", 8, 2, 1072, 4096, 274432),
    # 8 * 196 = 1568 = 2^5 * 7^2 -> 2^12 * 49
    ("turboquant_k8v4", 8, 2, 1568, 4096, 200704),
    # 4 * 102 = 408 = 2^3 * 3 * 17; 2 * 4 * 128 * 2 = 2048 = 2^11 -> 2^11 * 51
    ("turboquant_3bit_nc", 4, 2, 408, 2048, 104448),
    # fp32 skip layers: 2 * 8 * 128 * 4 = 8192 = 2^13; 8 * 118 = 944 = 2^4 * 59
    ("turboquant_k3v4_nc", 8, 4, 944, 8192, 483328),
])
def test_attention_page_sizes(preset, hkv, dtype_bytes, tq, skip, want):
    cfg = C.from_cache_dtype(preset, 128)
    assert OC.tq_page_bytes_1_token(cfg, hkv) == tq
    assert OC.skip_page_bytes_1_token(128, hkv, dtype_bytes) == skip
    got = OC.attn_page_bytes_1_token(cfg, hkv, dtype_bytes)
    assert got == want
    assert got % tq == 0 and got % skip == 0 and got <= tq * skip
    assert OC.attn_page_bytes_1_token(cfg, hkv) == tq      # no skip layers: the TQ page


def _bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def test_ring_end_state_equals_direct_append():
    """40 decode steps through a 16-token ring: the compressed history is byte
    for byte what appending the same tokens directly writes, every token sits
    exactly once (compressed or in the ring), in order."""
    cfg = C.TQConfig(head_dim=64, key_quant_bits=3, value_quant_bits=4, norm_correction=True)
    hkv, cap, bs, steps = 2, 16, 16, 40
    rng = np.random.default_rng(12)
    pre = [20, 0]            # compressed tokens before the first step
    ring0 = [0, 5]           # ring tokens before the first step
    total = [pre[b] + ring0[b] + steps for b in range(2)]
    k_all = [_bf16(rng.standard_normal((total[b], hkv, 64))) for b in range(2)]
    v_all = [_bf16(rng.standard_normal((total[b], hkv, 64))) for b in range(2)]
    nblk = [math.ceil(t / bs) for t in total]
    tables = np.zeros((2, max(nblk)), np.int32)
    perm = rng.permutation(sum(nblk))
    tables[0, :nblk[0]] = perm[:nblk[0]]
    tables[1, :nblk[1]] = perm[nblk[0]:]
    pool = np.zeros((sum(nblk), hkv, bs, cfg.slot_size_aligned), np.uint8)
    ring_k = np.zeros((2, hkv, cap, 64), np.float32)
    ring_v = np.zeros_like(ring_k)
    for b in range(2):
        pos = np.arange(pre[b])
        OX.append(pool, k_all[b][:pre[b]], v_all[b][:pre[b]], tables[b, pos // bs] * bs + pos % bs, cfg, 0)
        ring_k[b, :, :ring0[b]] = np.transpose(k_all[b][pre[b]:pre[b] + ring0[b]], (1, 0, 2))
        ring_v[b, :, :ring0[b]] = np.transpose(v_all[b][pre[b]:pre[b] + ring0[b]], (1, 0, 2))
    st = OC.RingState(cfg, 0, pool, tables, pre, ring_k, ring_v, ring0)
    for s in range(steps):
        kn = np.stack([k_all[b][pre[b] + ring0[b] + s] for b in range(2)])
        vn = np.stack([v_all[b][pre[b] + ring0[b] + s] for b in range(2)])
        st.step(kn, vn)
        assert (st.ring_lens >= 1).all() and (st.ring_lens <= cap).all()
    direct = np.zeros_like(pool)
    for b in range(2):
        nc = int(st.seq_lens[b])
        assert nc + int(st.ring_lens[b]) == total[b]
        assert nc % cap == pre[b] % cap       # whole chunks only
        pos = np.arange(nc)
        OX.append(direct, k_all[b][:nc], v_all[b][:nc], tables[b, pos // bs] * bs + pos % bs, cfg, 0)
        r = int(st.ring_lens[b])
        assert np.array_equal(st.ring_k[b, :, :r], np.transpose(k_all[b][nc:], (1, 0, 2)))
        assert np.array_equal(st.ring_v[b, :, :r], np.transpose(v_all[b][nc:], (1, 0, 2)))
    assert np.array_equal(st.pool, direct)
    # sequence 0: flushes at steps 17 and 33; sequence 1 (5 ring tokens first): at steps 12 and 28
    assert list(st.seq_lens) == [52, 32] and list(st.ring_lens) == [8, 13]
