"""Pins of the oracle's decode attention: brute force, closed forms, a library
routine (torch scaled_dot_product_attention on CPU, float64) and the
rotated-query identity the fused kernel relies on."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import codec as X
from oracle import config as C


def _fill(cfg, lens, hkv, bs=16, seed=0, layer=0, extra_blocks=3):
    rng = np.random.default_rng(seed)
    nblk_seq = [math.ceil(n / bs) for n in lens]
    nb = sum(nblk_seq) + extra_blocks
    perm = rng.permutation(nb)
    maxb = max(max(nblk_seq), 1)
    tables = np.zeros((len(lens), maxb), np.int32)
    pool = np.zeros((nb, hkv, bs, cfg.slot_size_aligned), np.uint8)
    used = 0
    for b, n in enumerate(lens):
        tables[b, :nblk_seq[b]] = perm[used:used + nblk_seq[b]]
        used += nblk_seq[b]
        if n == 0:
            continue
        k = rng.standard_normal((n, hkv, cfg.head_dim)).astype(np.float32)
        v = rng.standard_normal((n, hkv, cfg.head_dim)).astype(np.float32)
        X.append(pool, k, v, X.logical_slot_ids(tables[b], n, bs), cfg, layer)
    return pool, tables


def _brute(q, pool, tables, lens, cfg, layer, scale):
    """Pure-Python loops over tokens (tiny inputs only)."""
    b_s, hq, d = q.shape
    hkv = pool.shape[1]
    g = hq // hkv
    bs = pool.shape[2]
    out = np.zeros_like(q, dtype=np.float64)
    for b in range(b_s):
        for head in range(hq):
            h = head // g
            ks, vs = [], []
            for pos in range(lens[b]):
                sl = tables[b][pos // bs] * bs + pos % bs
                kk, vv = X.dequant_f64(X.gather_slots(pool, [sl], h), cfg, layer)
                ks.append(kk[0])
                vs.append(vv[0])
            if not ks:
                continue
            scores = [scale * sum(float(q[b, head, j]) * float(kk[j]) for j in range(d)) for kk in ks]
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for j in range(d):
                out[b, head, j] = sum(w[t] * vs[t][j] for t in range(len(ks))) / tot
    return out


@pytest.mark.parametrize("preset,d", [("turboquant_3bit_nc", 64), ("turboquant_k8v4", 64), ("turboquant_k3v4_nc", 96),
                                      ((3, 2), 128), ((8, 2), 64)])
def test_brute_force_tiny(preset, d):
    if isinstance(preset, tuple):  # 2-bit values
        cfg = C.TQConfig(head_dim=d, key_quant_bits=preset[0], value_quant_bits=preset[1], norm_correction=True)
    else:
        cfg = C.from_cache_dtype(preset, d)
    lens = [0, 5, 21]
    pool, tables = _fill(cfg, lens, hkv=2, seed=1)
    q = np.random.default_rng(2).standard_normal((3, 4, d)).astype(np.float32)
    got = A.decode_attention(q, pool, tables, lens, cfg, 0)
    want = _brute(q, pool, tables, lens, cfg, 0, 1 / math.sqrt(d))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    assert (got[0] == 0).all()


def test_single_token_returns_its_value():
    cfg = C.TQConfig(head_dim=64, key_quant_bits=3, value_quant_bits=4)
    pool, tables = _fill(cfg, [1], hkv=2, seed=3)
    q = np.random.default_rng(4).standard_normal((1, 4, 64))
    out = A.decode_attention(q, pool, tables, [1], cfg, 0)
    for h in range(2):
        _, v = X.dequant_f64(X.gather_slots(pool, [tables[0][0] * 16], h), cfg, 0)
        assert np.array_equal(out[0, 2 * h], v[0]) and np.array_equal(out[0, 2 * h + 1], v[0])


def test_identical_keys_average_values():
    cfg = C.TQConfig(head_dim=64, key_quant_bits=4, value_quant_bits=4)
    n = 20
    rng = np.random.default_rng(5)
    k = np.repeat(rng.standard_normal((1, 1, 64)).astype(np.float32), n, axis=0)
    v = rng.standard_normal((n, 1, 64)).astype(np.float32)
    pool = np.zeros((2, 1, 16, cfg.slot_size_aligned), np.uint8)
    X.append(pool, k, v, np.arange(n), cfg, 0)
    q = rng.standard_normal((1, 2, 64))
    out = A.decode_attention(q, pool, np.array([[0, 1]]), [n], cfg, 0)
    _, vhat = X.dequant_f64(X.gather_slots(pool, np.arange(n), 0), cfg, 0)
    assert np.allclose(out[0], vhat.mean(0)[None, :].repeat(2, 0), rtol=1e-12, atol=1e-14)


def test_ring_only_matches_torch_sdpa():
    cfg = C.from_cache_dtype("turboquant_3bit_nc", 128)
    b_s, hkv, hq, cap = 2, 2, 8, 128
    rng = np.random.default_rng(6)
    ring_k = torch.from_numpy(rng.standard_normal((b_s, hkv, cap, 128)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ring_v = torch.from_numpy(rng.standard_normal((b_s, hkv, cap, 128)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ring_lens = np.array([128, 37])
    q = rng.standard_normal((b_s, hq, 128))
    pool = np.zeros((1, hkv, 16, cfg.slot_size_aligned), np.uint8)
    out = A.decode_attention(q, pool, np.zeros((b_s, 1), np.int32), [0, 0], cfg, 0,
                             ring_k=ring_k, ring_v=ring_v, ring_lens=ring_lens)
    for b in range(b_s):
        r = ring_lens[b]
        kk = torch.from_numpy(ring_k[b, :, :r]).double().repeat_interleave(hq // hkv, dim=0)
        vv = torch.from_numpy(ring_v[b, :, :r]).double().repeat_interleave(hq // hkv, dim=0)
        qq = torch.from_numpy(q[b]).double()[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0, :].numpy()
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_compressed_plus_ring_equals_concatenated_sdpa():
    cfg = C.from_cache_dtype("turboquant_k3v4_nc", 96)
    lens = [30]
    pool, tables = _fill(cfg, lens, hkv=2, seed=7)
    rng = np.random.default_rng(8)
    ring_k = rng.standard_normal((1, 2, 16, 96))
    ring_v = rng.standard_normal((1, 2, 16, 96))
    q = rng.standard_normal((1, 4, 96))
    out = A.decode_attention(q, pool, tables, lens, cfg, 1, ring_k, ring_v, np.array([9]), scale=0.3)
    for h in range(2):
        k, v = A.sequence_kv(pool, tables[0], 30, h, cfg, 1)
        kk = torch.from_numpy(np.concatenate([k, ring_k[0, h, :9]]))[None].repeat(2, 1, 1)
        vv = torch.from_numpy(np.concatenate([v, ring_v[0, h, :9]]))[None].repeat(2, 1, 1)
        qq = torch.from_numpy(q[0, 2 * h:2 * h + 2])[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.3)[:, 0].numpy()
        assert np.allclose(out[0, 2 * h:2 * h + 2], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("preset,d", [("turboquant_4bit_nc", 128), ("turboquant_3bit_nc", 128),
                                      ("turboquant_k3v4_nc", 96)])
@pytest.mark.parametrize("nc", [False, True])
def test_rotated_query_form_equals_dequantized_dot(preset, d, nc):
    base = C.from_cache_dtype(preset, d)
    cfg = C.TQConfig(head_dim=d, key_quant_bits=base.key_quant_bits,
                     value_quant_bits=base.value_quant_bits, norm_correction=nc)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((200, d)).astype(np.float32)
    slots = X.encode_slots(k, k, cfg, 4)
    q = rng.standard_normal(d)
    khat, _ = X.dequant_f64(slots, cfg, 4)
    direct = khat @ q
    rot = A.rotated_scores(q, slots, cfg, 4)
    assert np.allclose(rot, direct, rtol=1e-12, atol=1e-12 * np.abs(direct).max())


def test_gqa_mapping():
    cfg = C.TQConfig(head_dim=64, key_quant_bits=3, value_quant_bits=3)
    pool, tables = _fill(cfg, [40], hkv=2, seed=10)
    q = np.random.default_rng(11).standard_normal((1, 6, 64))
    out = A.decode_attention(q, pool, tables, [40], cfg, 0)
    # query heads 0-2 read kv head 0, 3-5 read kv head 1
    for g in range(6):
        k, v = A.sequence_kv(pool, tables[0], 40, g // 3, cfg, 0)
        s = (k @ q[0, g]) / 8.0
        p = np.exp(s - s.max())
        assert np.allclose(out[0, g], (p / p.sum()) @ v, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- continuation prefill

def test_prefill_one_token_chunk_is_decode_with_one_ring_token():
    """A one-token chunk attends to the history plus itself: exactly decode
    with that token as the only ring token."""
    cfg = C.from_cache_dtype("turboquant_k3v4_nc", 96)
    lens = [37, 0, 16]
    pool, tables = _fill(cfg, lens, hkv=2, seed=21)
    rng = np.random.default_rng(22)
    q = rng.standard_normal((3, 4, 96))
    kc = rng.standard_normal((3, 2, 96))
    vc = rng.standard_normal((3, 2, 96))
    got = A.prefill_attention(q, kc, vc, [0, 1, 2, 3], pool, tables, lens, cfg, 1)
    want = A.decode_attention(q, pool, tables, lens, cfg, 1, ring_k=kc[:, :, None], ring_v=vc[:, :, None],
                              ring_lens=[1, 1, 1])
    assert np.array_equal(got, want)


def test_prefill_without_history_is_causal_sdpa():
    """No compressed history: causal attention over the chunk, checked with
    torch's scaled_dot_product_attention (is_causal) in float64."""
    cfg = C.from_cache_dtype("turboquant_4bit_nc", 64)
    pool = np.zeros((1, 2, 16, cfg.slot_size_aligned), np.uint8)
    rng = np.random.default_rng(23)
    n = 19
    q = rng.standard_normal((n, 6, 64))
    kc = rng.standard_normal((n, 2, 64))
    vc = rng.standard_normal((n, 2, 64))
    got = A.prefill_attention(q, kc, vc, [0, n], pool, np.zeros((1, 1), np.int32), [0], cfg, 0, scale=0.2)
    qq = torch.from_numpy(q).permute(1, 0, 2)                                  # [6, n, 64]
    kk = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(3, dim=0)     # head g -> kv head g // 3
    vv = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(3, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=0.2)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_brute_force_tiny():
    """Two sequences with history and chunks of 3 and 5 tokens: every output
    row against an explicit loop over the visible keys."""
    cfg = C.TQConfig(head_dim=64, key_quant_bits=4, value_quant_bits=2, norm_correction=True)
    lens = [21, 5]
    pool, tables = _fill(cfg, lens, hkv=1, seed=24)
    rng = np.random.default_rng(25)
    cu = [0, 3, 8]
    q = rng.standard_normal((8, 2, 64))
    kc = rng.standard_normal((8, 1, 64))
    vc = rng.standard_normal((8, 1, 64))
    got = A.prefill_attention(q, kc, vc, cu, pool, tables, lens, cfg, 2)
    sc = 1 / math.sqrt(64)
    for b in range(2):
        kh, vh = A.sequence_kv(pool, tables[b], lens[b], 0, cfg, 2)
        for t in range(cu[b + 1] - cu[b]):
            row = cu[b] + t
            keys = list(kh) + [kc[cu[b] + j, 0] for j in range(t + 1)]
            vals = list(vh) + [vc[cu[b] + j, 0] for j in range(t + 1)]
            for g in range(2):
                s = np.array([sc * float(np.dot(q[row, g], k)) for k in keys])
                w = np.exp(s - s.max())
                w /= w.sum()
                assert np.allclose(got[row, g], sum(wi * vi for wi, vi in zip(w, vals)), rtol=1e-11, atol=1e-12)
