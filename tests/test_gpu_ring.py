"""GPU parity of the device-side ring manager: tq_ring_flush + tq_ring_append
over many decode steps leave the pool bytes, the ring contents and the
lengths exactly where the oracle's ring leaves them, and a decode over the
result matches the oracle's attention."""

import math

import numpy as np
import pytest

from oracle import attention as OA
from oracle import cache as OCache
from oracle import codec as OX
from tests.gpu_common import ATTN_RTOL, announce, oracle_cfg, per_head_rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")


@pytest.mark.parametrize("d,kb,vb,cap,steps", [(128, 3, 3, 128, 300), (64, 4, 2, 16, 50), (96, 8, 4, 32, 70)])
def test_ring_steps_match_oracle(d, kb, vb, cap, steps):
    announce(f"ring steps d={d} kb={kb} vb={vb} cap={cap} steps={steps}")
    cfg = tq.config_init(d, kb, vb, True, 42)
    ocfg = oracle_cfg(cfg)
    hkv, hq, bs, layer = 2, 8, 16, 3
    rng = np.random.default_rng(d + cap)
    pre = [37, 0, 16, 5]          # compressed tokens before the first step
    ring0 = [0, cap - 3, cap, 1]  # ring tokens before it (one full ring)
    B = len(pre)
    total = [pre[b] + ring0[b] + steps for b in range(B)]
    toks_k = [torch.from_numpy(rng.standard_normal((total[b], hkv, d)).astype(np.float32)).to(torch.bfloat16)
              for b in range(B)]
    toks_v = [torch.from_numpy(rng.standard_normal((total[b], hkv, d)).astype(np.float32)).to(torch.bfloat16)
              for b in range(B)]
    kf = [t.float().numpy() for t in toks_k]
    vf = [t.float().numpy() for t in toks_v]
    nblk = [math.ceil(t / bs) for t in total]
    tables = np.zeros((B, max(nblk)), np.int32)
    perm = rng.permutation(sum(nblk))
    o = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    pool_np = np.zeros((sum(nblk), hkv, bs, cfg.slot_size_aligned), np.uint8)
    ring_k = torch.zeros((B, hkv, cap, d), dtype=torch.bfloat16)
    ring_v = torch.zeros_like(ring_k)
    for b in range(B):
        pos = np.arange(pre[b])
        OX.append(pool_np, kf[b][:pre[b]], vf[b][:pre[b]], tables[b, pos // bs] * bs + pos % bs, ocfg, layer)
        ring_k[b, :, :ring0[b]] = toks_k[b][pre[b]:pre[b] + ring0[b]].transpose(0, 1)
        ring_v[b, :, :ring0[b]] = toks_v[b][pre[b]:pre[b] + ring0[b]].transpose(0, 1)
    ost = OCache.RingState(ocfg, layer, pool_np.copy(), tables, pre, ring_k.float().numpy(), ring_v.float().numpy(),
                           ring0)
    g_pool = torch.from_numpy(pool_np).cuda()
    g_rk, g_rv = ring_k.cuda(), ring_v.cuda()
    g_rl = torch.tensor(ring0, dtype=torch.int32, device="cuda")
    g_sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    g_tab = torch.from_numpy(tables).cuda()
    for s in range(steps):
        kn = torch.stack([toks_k[b][pre[b] + ring0[b] + s] for b in range(B)])
        vn = torch.stack([toks_v[b][pre[b] + ring0[b] + s] for b in range(B)])
        tq.ring_step(cfg, layer, kn.cuda(), vn.cuda(), g_rk, g_rv, g_rl, g_sl, g_tab, g_pool)
        ost.step(kn.float().numpy(), vn.float().numpy())
    torch.cuda.synchronize()
    assert g_rl.cpu().tolist() == [int(x) for x in ost.ring_lens]
    assert g_sl.cpu().tolist() == [int(x) for x in ost.seq_lens]
    got = g_pool.cpu().numpy()
    mism = np.argwhere(got != ost.pool)
    assert mism.size == 0, f"{len(mism)} pool bytes differ; first at {mism[:4].tolist()}"
    rk = g_rk.float().cpu().numpy()
    for b in range(B):
        r = int(ost.ring_lens[b])
        assert np.array_equal(rk[b, :, :r], ost.ring_k[b, :, :r])
    # decode over the compressed history plus the ring
    q = torch.from_numpy(rng.standard_normal((B, hq, d)).astype(np.float32)).to(torch.bfloat16)
    lens = [int(x) for x in ost.seq_lens]
    out = tq.decode_attention(cfg, layer, q.cuda(), g_pool, g_tab, g_sl, max(lens), ring_k=g_rk, ring_v=g_rv,
                              ring_lens=g_rl)
    want = OA.decode_attention(q.float().numpy(), ost.pool, tables, lens, ocfg, layer, ring_k=ost.ring_k,
                               ring_v=ost.ring_v, ring_lens=ost.ring_lens.astype(np.int32))
    err = per_head_rel_l2(out.cpu().numpy(), want)
    announce(f"  decode rel L2 {err:.2e}")
    assert err <= ATTN_RTOL


def test_ring_flush_leaves_partial_rings_alone():
    announce("ring flush partial rings")
    cfg = tq.config_from_preset("turboquant_k3v4_nc", 128)
    B, hkv, cap, bs = 3, 2, 128, 16
    pool = torch.zeros((40, hkv, bs, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    tables = torch.arange(40, dtype=torch.int32, device="cuda").view(1, 40).repeat(B, 1).contiguous()
    rk = torch.randn((B, hkv, cap, 128), device="cuda").to(torch.bfloat16)
    rv = torch.randn_like(rk)
    rl = torch.tensor([127, 0, 5], dtype=torch.int32, device="cuda")
    sl = torch.tensor([0, 16, 32], dtype=torch.int32, device="cuda")
    tq.ring_flush(cfg, 0, rk, rv, rl, sl, tables, pool)
    torch.cuda.synchronize()
    assert rl.cpu().tolist() == [127, 0, 5] and sl.cpu().tolist() == [0, 16, 32]
    assert int(pool.count_nonzero()) == 0
