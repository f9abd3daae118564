"""GPU parity of continuation prefill over the compressed cache against the
oracle's float64 definition (history dequantized, chunk exact and causal):
relative L2 <= 2e-3 per (chunk row, query head)."""

import math

import numpy as np
import pytest

from oracle import attention as OA
from oracle import codec as OX
from tests.gpu_common import ATTN_RTOL, announce, oracle_cfg, oracle_pool, per_head_rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

CASES = {
    # name: (d, kb, vb, nc, hq, hkv, hist_lens, chunk_lens, q dtype[, block size])
    "4bit_nc_g4": (128, 4, 4, True, 8, 2, [300, 0], [37, 5], "bf16"),
    "k3v4_d96_g8": (96, 3, 4, True, 16, 2, [1500, 17], [64, 1], "bf16"),
    "k8v2_d64_g1": (64, 8, 2, False, 2, 2, [40], [100], "f32"),
    "3bit_g16_f16": (128, 3, 3, True, 32, 2, [700, 129, 0], [9, 16, 33], "f16"),
    # 48-token blocks: the history walk wraps blocks at offsets that are not
    # powers of two
    "4bit_bs48": (128, 4, 4, True, 8, 2, [700, 130], [20, 3], "bf16", 48),
    # 5000 history tokens with few rows: four history splits of 1280 tokens,
    # the last one ragged (1160)
    "3bit_splits": (128, 3, 4, True, 8, 2, [5000], [40], "bf16"),
}


def _scenario(d, kb, vb, nc, hq, hkv, hist, chunks, qdt, seed, bs=16):
    cfg = tq.config_init(d, kb, vb, nc, 42)
    ocfg = oracle_cfg(cfg)
    rng = np.random.default_rng(seed)
    B = len(hist)
    nblk = [max(1, math.ceil(n / bs)) for n in hist]
    nb = sum(nblk) + 1
    perm = rng.permutation(nb)
    tables = np.zeros((B, max(nblk)), np.int32)
    o = 0
    ks, vs, maps = [], [], []
    for b, n in enumerate(hist):
        tables[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        k[:, :, rng.choice(d, 4, replace=False)] *= 10
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
        v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
        pos = np.arange(n)
        maps.append(tables[b, pos // bs].astype(np.int64) * bs + pos % bs)
        ks.append(k)
        vs.append(v)
    pool = oracle_pool(ocfg, 0, np.concatenate(ks), np.concatenate(vs), np.concatenate(maps), nb, hkv, bs)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    n = int(cu[-1])
    q = torch.from_numpy(rng.standard_normal((n, hq, d)).astype(np.float32)).to(DT[qdt])
    kc = torch.from_numpy(rng.standard_normal((n, hkv, d)).astype(np.float32)).to(torch.bfloat16)
    vc = torch.from_numpy(rng.standard_normal((n, hkv, d)).astype(np.float32)).to(torch.bfloat16)
    return cfg, ocfg, pool, tables, cu, q, kc, vc


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name):
    d, kb, vb, nc, hq, hkv, hist, chunks, qdt, *bs = CASES[name]
    announce(f"prefill {name}")
    cfg, ocfg, pool, tables, cu, q, kc, vc = _scenario(d, kb, vb, nc, hq, hkv, hist, chunks, qdt, sum(name.encode()), *bs)
    out = tq.prefill_attention(cfg, 0, q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(cu).cuda(), max(chunks),
                               torch.from_numpy(pool).cuda(), torch.from_numpy(tables).cuda(),
                               torch.tensor(hist, dtype=torch.int32).cuda(), max(hist))
    want = OA.prefill_attention(q.float().numpy(), kc.float().numpy(), vc.float().numpy(), cu, pool, tables, hist,
                                ocfg, 0)
    err = per_head_rel_l2(out.cpu().numpy(), want)  # rows x heads
    announce(f"  rel L2 {err:.2e}")
    assert err <= ATTN_RTOL


def test_prefill_garbage_workspace_and_repeat():
    """Workspace contents on entry do not matter; repeated calls agree bit for bit."""
    d, kb, vb, nc, hq, hkv, hist, chunks, qdt, *_ = CASES["4bit_nc_g4"]
    announce("prefill garbage workspace")
    cfg, ocfg, pool, tables, cu, q, kc, vc = _scenario(d, kb, vb, nc, hq, hkv, hist, chunks, qdt, 5)
    args = (q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(cu).cuda(), max(chunks), torch.from_numpy(pool).cuda(),
            torch.from_numpy(tables).cuda(), torch.tensor(hist, dtype=torch.int32).cuda(), max(hist))
    need = tq.prefill_workspace_size(cfg, len(hist), hq, hkv, max(chunks), max(hist), tables.shape[1], tq.BF16)
    outs = []
    for fill in (0xff, 0x41, 0x00):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        outs.append(tq.prefill_attention(cfg, 0, *args, workspace=ws).cpu().numpy())
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))


@pytest.mark.timeout(900)
def test_prefill_full_size_sampled():
    """The continuation-prefill workload at full size (4 sequences x 32768
    compressed history tokens + 512-token chunks, D=128, 32 q / 8 KV heads),
    with the inputs and launch bench.py times: sampled rows (first, second,
    middle and last chunk token of the first and last sequence, all query
    heads) against the oracle's definition, row by row (the sequence's
    dequantized history plus the chunk's exact tokens 0..t)."""
    from workloads import WORKLOADS, KVSource
    from workloads import gpu as WG

    w = WORKLOADS["prefill_4bit_nc"]
    picks = (0, w.batch - 1)
    announce(f"prefill full size {w.name}: sequences {picks}")
    built = WG.build(w, "cuda", n_pools=1, capture=picks, extra_blocks=w.batch * -(-w.chunk // w.block_size))
    n = w.batch * w.chunk
    ck, cv = KVSource(w, "cuda", stream_id=55).kv(n)
    cq = KVSource(w, "cuda", stream_id=56).q(n)
    cu = torch.arange(0, n + 1, w.chunk, dtype=torch.int32, device="cuda")
    out = tq.prefill_attention(built.cfg, 0, cq, ck, cv, cu, w.chunk, built.pools[0], built.tables, built.seq_lens,
                               built.max_seq_len)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ocfg = oracle_cfg(built.cfg)
    q = cq.float().cpu().numpy()
    kc = ck.float().cpu().numpy()
    vc = cv.float().cpu().numpy()
    bs = w.block_size
    grp = w.num_q_heads // w.num_kv_heads
    scale = 1.0 / math.sqrt(w.head_dim)
    worst = 0.0
    for b in picks:
        kh_src, vh_src = built.captured[b]
        m = kh_src.shape[0]
        nblk = max(1, -(-m // bs))
        opool = np.zeros((nblk, w.num_kv_heads, bs, ocfg.slot_size_aligned), np.uint8)
        for s0 in range(0, m, 16384):
            s1 = min(m, s0 + 16384)
            OX.append(opool, kh_src[s0:s1], vh_src[s0:s1], np.arange(s0, s1), ocfg, 0)
        table = np.arange(nblk, dtype=np.int32)
        r0 = b * w.chunk
        for h in range(w.num_kv_heads):
            kh, vh = OA.sequence_kv(opool, table, m, h, ocfg, 0)
            for t in (0, 1, w.chunk // 2, w.chunk - 1):
                k = np.concatenate([kh, kc[r0:r0 + t + 1, h].astype(np.float64)], axis=0)
                v = np.concatenate([vh, vc[r0:r0 + t + 1, h].astype(np.float64)], axis=0)
                want = OA.softmax_attend(q[r0 + t, h * grp:(h + 1) * grp].astype(np.float64), k, v, scale)
                worst = max(worst, per_head_rel_l2(got[r0 + t:r0 + t + 1, h * grp:(h + 1) * grp], want[None]))
    announce(f"  sampled rows: max rel L2 {worst:.2e}")
    assert worst <= ATTN_RTOL


def test_prefill_invalid_block_ids_skip_their_tokens():
    """History blocks outside the pool (past num_blocks, or negative) are
    read as nothing: their tokens are masked for every row, and each row
    attends to the rest of the history plus its causal chunk tokens."""
    announce("prefill invalid block ids")
    hist, chunks = [300, 70], [10, 5]
    cfg, ocfg, pool, tables, cu, q, kc, vc = _scenario(128, 4, 4, True, 8, 2, hist, chunks, "bf16", 44)
    nb, hkv, bs = pool.shape[0], pool.shape[1], pool.shape[2]
    bad = tables.copy()
    bad[0, 2] = nb + 3   # past the pool
    bad[1, 1] = -5       # negative
    drop = {0: {2}, 1: {1}}
    out = tq.prefill_attention(cfg, 0, q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(cu).cuda(), max(chunks),
                               torch.from_numpy(pool).cuda(), torch.from_numpy(bad).cuda(),
                               torch.tensor(hist, dtype=torch.int32).cuda(), max(hist))
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    qf = q.float().numpy().astype(np.float64)
    kcf = kc.float().numpy().astype(np.float64)
    vcf = vc.float().numpy().astype(np.float64)
    g = q.shape[1] // hkv
    want = np.zeros(got.shape, np.float64)
    for b in range(len(hist)):
        keep = np.array([(t // bs) not in drop[b] for t in range(hist[b])], bool)
        r0, r1 = int(cu[b]), int(cu[b + 1])
        for h in range(hkv):
            kh, vh = OA.sequence_kv(pool, tables[b], hist[b], h, ocfg, 0)
            for t in range(r1 - r0):
                k = np.concatenate([kh[keep], kcf[r0:r0 + t + 1, h]])
                v = np.concatenate([vh[keep], vcf[r0:r0 + t + 1, h]])
                want[r0 + t, h * g:(h + 1) * g] = OA.softmax_attend(qf[r0 + t, h * g:(h + 1) * g], k, v,
                                                                    1.0 / math.sqrt(q.shape[2]))
    err = per_head_rel_l2(got, want)
    announce(f"  rel L2 {err:.2e}")
    assert err <= ATTN_RTOL
