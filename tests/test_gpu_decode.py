"""GPU parity: fused decode attention against the oracle's float64 attention
over the dequantized cache (relative L2 <= 2e-3 per sequence and query
head), on pools the oracle encodes itself and uploads."""

import math

import numpy as np
import pytest

from oracle import attention as OA
from tests.gpu_common import ATTN_RTOL, announce, oracle_cfg, oracle_pool, per_head_rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _scenario(d, kb, vb, nc, hq, hkv, lens, ring_lens=None, ring_cap=0, bs=16, seed=0, qdt="bf16",
              outliers=True, layer=0):
    cfg = tq.config_init(d, kb, vb, nc, 42)
    ocfg = oracle_cfg(cfg)
    rng = np.random.default_rng(seed)
    b_s = len(lens)
    nblk = [max(1, math.ceil(n / bs)) for n in lens]
    nb = sum(nblk) + 2
    perm = rng.permutation(nb)
    tables = np.zeros((b_s, max(nblk)), np.int32)
    used = 0
    ks, vs, maps = [], [], []
    for b, n in enumerate(lens):
        tables[b, :nblk[b]] = perm[used:used + nblk[b]]
        used += nblk[b]
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        if outliers:
            k[:, :, rng.choice(d, 4, replace=False)] *= 10
            v[:, :, rng.choice(d, 4, replace=False)] *= 10
        k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
        v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
        pos = np.arange(n)
        maps.append(tables[b, pos // bs].astype(np.int64) * bs + pos % bs)
        ks.append(k)
        vs.append(v)
    kk = np.concatenate(ks) if ks else np.zeros((0, hkv, d), np.float32)
    vv = np.concatenate(vs) if vs else np.zeros((0, hkv, d), np.float32)
    pool_np = oracle_pool(ocfg, layer, kk, vv, np.concatenate(maps), nb, hkv, bs)
    q = torch.from_numpy(rng.standard_normal((b_s, hq, d)).astype(np.float32)).to(DT[qdt])
    ring = None
    if ring_cap:
        rk = torch.from_numpy(rng.standard_normal((b_s, hkv, ring_cap, d)).astype(np.float32)).to(torch.bfloat16)
        rv = torch.from_numpy(rng.standard_normal((b_s, hkv, ring_cap, d)).astype(np.float32)).to(torch.bfloat16)
        ring = (rk, rv, np.asarray(ring_lens, np.int32))
    return cfg, ocfg, pool_np, tables, q, ring


def _run(cfg, ocfg, pool_np, tables, lens, q, ring, split_tokens=0, layer=0, scale=0.0):
    pool = torch.from_numpy(pool_np).cuda()
    kw = {}
    if ring is not None:
        kw = dict(ring_k=ring[0].cuda(), ring_v=ring[1].cuda(), ring_lens=torch.from_numpy(ring[2]).cuda())
    out = tq.decode_attention(cfg, layer, q.cuda(), pool, torch.from_numpy(tables).cuda(),
                              torch.tensor(lens, dtype=torch.int32).cuda(), max(lens) if len(lens) else 0,
                              softmax_scale=scale, split_tokens=split_tokens, **kw)
    got = out.cpu().numpy()
    want = OA.decode_attention(q.float().numpy(), pool_np, tables, lens, ocfg, layer,
                               ring_k=None if ring is None else ring[0].float().numpy(),
                               ring_v=None if ring is None else ring[1].float().numpy(),
                               ring_lens=None if ring is None else ring[2],
                               scale=scale if scale > 0 else None)
    return got, want


SCEN = {
    # name: (d, kb, vb, nc, hq, hkv, lens, ring_lens, ring_cap)
    "k8v4": (128, 8, 4, False, 32, 8, [1000, 17, 0], None, 0),
    "4bit_nc": (128, 4, 4, True, 32, 8, [2049, 300], None, 0),
    "4bit": (128, 4, 4, False, 8, 2, [333, 16, 15], None, 0),
    "3bit_nc_ring": (128, 3, 3, True, 64, 8, [700, 0, 33], [128, 5, 0], 128),
    "k3v4_nc_d96": (96, 3, 4, True, 16, 4, [1500, 16, 15, 1], None, 0),
    "d64_k3v4": (64, 3, 4, False, 4, 2, [512], None, 0),
    "d96_k8v3": (96, 8, 3, False, 12, 4, [257, 64], None, 0),
    "d64_k4v3_ring": (64, 4, 3, True, 6, 2, [95, 40], [17, 128], 128),
    # ring capacity not a multiple of the 32-token ring chunk; full chunks,
    # a partial second chunk and a ring-only sequence
    "d96_k3v4_ring100": (96, 3, 4, True, 16, 4, [50, 300, 0], [100, 70, 64], 100),
    # 2-bit values at each column packing (G = 4, 8, 16 query heads per KV head)
    "k3v2_nc": (128, 3, 2, True, 32, 8, [1500, 31, 0], None, 0),
    "k4v2_g8_ring": (128, 4, 2, True, 16, 2, [600, 17], [40, 128], 128),
    "d96_k8v2": (96, 8, 2, False, 12, 4, [257, 64], None, 0),
    "d64_k3v2_g16": (64, 3, 2, True, 32, 2, [400], None, 0),
}


@pytest.mark.parametrize("name", list(SCEN))
@pytest.mark.parametrize("split", [0, 64])
def test_decode_matches_oracle(name, split):
    d, kb, vb, nc, hq, hkv, lens, rl, rc = SCEN[name]
    announce(f"decode {name} split={split}")
    cfg, ocfg, pool_np, tables, q, ring = _scenario(d, kb, vb, nc, hq, hkv, lens, rl, rc, seed=sum(name.encode()))
    got, want = _run(cfg, ocfg, pool_np, tables, lens, q, ring, split_tokens=split)
    err = per_head_rel_l2(got, want)
    announce(f"  rel L2 {err:.2e}")
    assert err <= ATTN_RTOL, err


def test_tiny_workload_end_to_end():
    """The tiny workload: GPU quantize (511 + 1 tokens) then decode over 512,
    against the oracle's own encode and attention."""
    from workloads import tiny_numpy
    announce("decode tiny workload")
    k, v, q = tiny_numpy()
    cfg = tq.config_init(64, 3, 4, False, 42)
    ocfg = oracle_cfg(cfg)
    pool = torch.zeros((32, 2, 16, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    ids = torch.arange(512, dtype=torch.int64, device="cuda")
    tq.quantize_append(cfg, 0, torch.from_numpy(k[:511]).cuda(), torch.from_numpy(v[:511]).cuda(), ids[:511], pool)
    tq.quantize_append(cfg, 0, torch.from_numpy(k[511:]).cuda(), torch.from_numpy(v[511:]).cuda(), ids[511:], pool)
    tables = np.arange(32, dtype=np.int32)[None]
    out = tq.decode_attention(cfg, 0, torch.from_numpy(q).cuda(), pool, torch.from_numpy(tables).cuda(),
                              torch.tensor([512], dtype=torch.int32).cuda(), 512)
    pool_np = oracle_pool(ocfg, 0, k, v, np.arange(512), 32, 2, 16)
    want = OA.decode_attention(q, pool_np, tables, [512], ocfg, 0)
    assert per_head_rel_l2(out.cpu().numpy(), want) <= ATTN_RTOL


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_gqa_group_sizes(g):
    announce(f"decode gqa g={g}")
    hkv = 2
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 3, 4, True, g * hkv, hkv, [300, 47], seed=g)
    got, want = _run(cfg, ocfg, pool_np, tables, [300, 47], q, ring)
    err = per_head_rel_l2(got, want)
    announce(f"  rel L2 {err:.2e}")
    assert err <= ATTN_RTOL


@pytest.mark.parametrize("qdt", ["f32", "f16"])
def test_query_dtypes(qdt):
    announce(f"decode q dtype {qdt}")
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 4, 4, True, 16, 4, [400], seed=3, qdt=qdt)
    got, want = _run(cfg, ocfg, pool_np, tables, [400], q, ring)
    assert per_head_rel_l2(got, want) <= ATTN_RTOL


@pytest.mark.parametrize("bs,split", [(32, 0), (64, 0), (48, 0), (48, 16), (80, 32)])
def test_block_sizes(bs, split):
    # 48 and 80 are not powers of two; with small splits the ranges start
    # inside a block, so the tile walk starts at an offset and wraps
    announce(f"decode block size {bs} split {split}")
    lens = [250, 64, 63]
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 3, 3, True, 16, 2, lens, bs=bs, seed=bs)
    got, want = _run(cfg, ocfg, pool_np, tables, lens, q, ring, split_tokens=split)
    assert per_head_rel_l2(got, want) <= ATTN_RTOL


def test_layer_and_scale():
    announce("decode layer 6 scale 0.05")
    lens = [200]
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 4, 4, True, 8, 2, lens, seed=21, layer=6)
    got, want = _run(cfg, ocfg, pool_np, tables, lens, q, ring, layer=6, scale=0.05)
    assert per_head_rel_l2(got, want) <= ATTN_RTOL


def test_layer_adaptive_key_bits():
    """Layer-adaptive key bits end to end: each layer's config from
    tq.layer_config (4-bit keys below layer 4, the base 3-bit keys from layer
    4), quantize-append on the GPU with that layer's signs, slot bytes equal to
    the oracle's layer_config encoding, decode within tolerance."""
    from oracle import config as OC
    base = tq.config_from_preset("turboquant_k3v4_nc", 128)
    obase = oracle_cfg(base)
    n, hkv, hq, bs = 300, 2, 8, 16
    rng = np.random.default_rng(33)
    k = torch.from_numpy(rng.standard_normal((n, hkv, 128)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((n, hkv, 128)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((1, hq, 128)).astype(np.float32)).to(torch.bfloat16)
    nblk = math.ceil(n / bs)
    tables = rng.permutation(nblk).astype(np.int32)[None]
    pos = np.arange(n)
    mapping = tables[0, pos // bs].astype(np.int64) * bs + pos % bs
    for layer, want_kb in ((2, 4), (4, 3)):
        announce(f"decode layer-adaptive layer={layer}")
        cfg = tq.layer_config(base, layer)
        ocfg = OC.layer_config(obase, layer)
        assert cfg.key_quant_bits == ocfg.key_quant_bits == want_kb
        pool = torch.zeros((nblk, hkv, bs, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
        tq.quantize_append(cfg, layer, k.cuda(), v.cuda(), torch.from_numpy(mapping).cuda(), pool)
        pool_np = oracle_pool(ocfg, layer, k.float().numpy(), v.float().numpy(), mapping, nblk, hkv, bs)
        assert np.array_equal(pool.cpu().numpy(), pool_np)
        out = tq.decode_attention(cfg, layer, q.cuda(), pool, torch.from_numpy(tables).cuda(),
                                  torch.tensor([n], dtype=torch.int32).cuda(), n)
        want = OA.decode_attention(q.float().numpy(), pool_np, tables, [n], ocfg, layer)
        assert per_head_rel_l2(out.cpu().numpy(), want) <= ATTN_RTOL


def split_difference_bound(kappa, n):
    """Largest relative L2 difference between two split choices of one
    (sequence, query head) that the decode arithmetic allows.

    The scores s_t do not depend on the split (the same f16 operands summed
    over D in the same MFMA order). What changes is (i) the running maximum
    each weight is taken against: p_t = exp2(s_t - m) rounds with v_exp_f32's
    1 ulp (2^-23 relative), the weight p_t s'_t is carried as f16 hi + lo
    parts (2^-22 relative); and (ii) the order of the fp32 sums over the
    tokens (partials, merge). Under the probabilistic rounding model a sum
    of n terms errs by at most lambda sqrt(n) u of the sum of magnitudes
    (u = 2^-24), taken with lambda = 2 for each of the two runs. Relative
    term errors e move the output by at most kappa e relative to its norm
    (kappa over the terms the kernel adds: centred codes times p s' and the
    zero terms z' + c0 s' times p), so the two runs differ by at most
    kappa (2 (2^-22 + 2^-23) + 4 sqrt(n) u)."""
    u = 2.0 ** -24
    return kappa * (2 * (2.0 ** -22 + 2.0 ** -23) + 4 * np.sqrt(n) * u)


def test_split_invariance_and_determinism():
    from tests.gpu_common import attention_conditioning, rel_l2
    announce("decode split invariance")
    lens = [1777, 900, 3]
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 4, 4, True, 16, 4, lens, [40, 128, 0], 128, seed=4)
    runs = [_run(cfg, ocfg, pool_np, tables, lens, q, ring, split_tokens=s) for s in (16, 64, 256, 2048)]
    outs = [r[0] for r in runs]
    # every split choice meets the oracle bound
    for got, want in runs:
        err = per_head_rel_l2(got, want)
        announce(f"  rel L2 {err:.2e}")
        assert err <= ATTN_RTOL
    # between themselves they differ within the bound the arithmetic allows
    kappa, n_tok = attention_conditioning(q.float().numpy(), pool_np, tables, lens, ocfg, 0,
                                          ring[0].float().numpy(), ring[1].float().numpy(), ring[2])
    for o in outs[1:]:
        worst = worst_ratio = 0.0
        for b in range(len(lens)):
            for g in range(o.shape[1]):
                d = rel_l2(o[b, g], outs[0][b, g])
                bound = split_difference_bound(kappa[b, g], n_tok[b])
                worst = max(worst, d)
                worst_ratio = max(worst_ratio, d / bound)
                assert d <= bound, (b, g, d, bound, kappa[b, g])
        announce(f"  split-to-split {worst:.2e} (at most {worst_ratio:.2f} of the per-head bound)")
    again = _run(cfg, ocfg, pool_np, tables, lens, q, ring, split_tokens=64)[0]
    assert np.array_equal(again.view(np.uint32), outs[1].view(np.uint32))


def test_workspace_contents_do_not_matter():
    """The result depends on the inputs only: a workspace holding NaN or
    finite garbage from earlier use gives the same outputs (every partial the
    merge reads is written in the same call), at one-tile and default split
    sizes, over repeated calls."""
    announce("decode garbage workspace")
    lens = [1777, 900, 3]
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 4, 4, True, 16, 4, lens, [40, 128, 0], 128, seed=4)
    pool = torch.from_numpy(pool_np).cuda()
    kw = dict(ring_k=ring[0].cuda(), ring_v=ring[1].cuda(), ring_lens=torch.from_numpy(ring[2]).cuda())
    qd, td, ld = q.cuda(), torch.from_numpy(tables).cuda(), torch.tensor(lens, dtype=torch.int32).cuda()
    want = OA.decode_attention(q.float().numpy(), pool_np, tables, lens, ocfg, 0, ring_k=ring[0].float().numpy(),
                               ring_v=ring[1].float().numpy(), ring_lens=ring[2])
    for split in (16, 0):
        need, _ = tq.decode_workspace_size(cfg, len(lens), 16, max(lens), 128, split)
        for fill in (0xff, 0x41, 0x7f) * 2:
            ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
            out = tq.decode_attention(cfg, 0, qd, pool, td, ld, max(lens), workspace=ws, split_tokens=split, **kw)
            err = per_head_rel_l2(out.cpu().numpy(), want)
            announce(f"  split={split} fill={fill:#x}: rel L2 {err:.2e}")
            assert err <= ATTN_RTOL


@pytest.mark.parametrize("split", [16, 0])
def test_repeated_calls_finite_and_identical(split):
    """Ranges that end inside a macro tile leave tile slots masked; their
    per-token scale and zero must not come from LDS left over by earlier
    workgroups (packed slot bytes read as floats can be Inf or NaN, and
    0 * NaN poisons a row). Ten calls in a row of FP8-key decode with many
    such ranges: every output finite, within tolerance, and bit-identical."""
    announce(f"decode repeated calls split={split}")
    lens = [1777, 900, 3, 0]
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 8, 4, False, 32, 8, lens, seed=44)
    pool = torch.from_numpy(pool_np).cuda()
    qd, td, ld = q.cuda(), torch.from_numpy(tables).cuda(), torch.tensor(lens, dtype=torch.int32).cuda()
    want = OA.decode_attention(q.float().numpy(), pool_np, tables, lens, ocfg, 0)
    outs = []
    for _ in range(10):
        out = tq.decode_attention(cfg, 0, qd, pool, td, ld, max(lens), split_tokens=split)
        outs.append(out.cpu().numpy())
    for i, o in enumerate(outs):
        assert np.isfinite(o).all(), f"call {i}: {int((~np.isfinite(o)).sum())} non-finite outputs"
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), f"call {i} differs"
    err = per_head_rel_l2(outs[0], want)
    announce(f"  rel L2 {err:.2e}")
    assert err <= ATTN_RTOL
    assert (outs[0][3] == 0).all()


def test_empty_context_gives_zeros():
    announce("decode empty")
    cfg = tq.config_from_preset("turboquant_3bit_nc", 128)
    pool = torch.zeros((1, 2, 16, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    q = torch.randn((3, 4, 128), device="cuda").to(torch.bfloat16)
    out = torch.full((3, 4, 128), 5.0, device="cuda")
    tq.decode_attention(cfg, 0, q, pool, torch.zeros((3, 1), dtype=torch.int32, device="cuda"),
                        torch.zeros(3, dtype=torch.int32, device="cuda"), 0, out=out)
    assert (out == 0).all()


def test_ring_only():
    announce("decode ring only")
    lens = [0, 0]
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 3, 3, True, 16, 2, lens, [128, 77], 128, seed=8)
    got, want = _run(cfg, ocfg, pool_np, tables, lens, q, ring)
    assert per_head_rel_l2(got, want) <= ATTN_RTOL


def test_invalid_block_ids_skip_their_tokens():
    """Block-table entries outside the pool (past num_blocks, or negative)
    make the kernel read none of their slots: their tokens are masked. The
    output is attention over the other tokens (the plain definition with
    those positions removed), finite, with no fault."""
    announce("decode invalid block ids")
    lens = [700, 300]
    cfg, ocfg, pool_np, tables, q, _ = _scenario(128, 4, 4, True, 8, 2, lens, seed=31)
    nb, hkv, bs = pool_np.shape[0], pool_np.shape[1], pool_np.shape[2]
    bad = tables.copy()
    bad[0, 3] = nb + 7   # past the pool
    bad[1, 0] = -1       # negative
    drop = {0: {3}, 1: {0}}  # logical blocks whose tokens are skipped
    out = tq.decode_attention(cfg, 0, q.cuda(), torch.from_numpy(pool_np).cuda(), torch.from_numpy(bad).cuda(),
                              torch.tensor(lens, dtype=torch.int32).cuda(), max(lens))
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    qf = q.float().numpy().astype(np.float64)
    g = q.shape[1] // hkv
    want = np.zeros(got.shape, np.float64)
    for b, n in enumerate(lens):
        keep = np.array([(t // bs) not in drop[b] for t in range(n)], bool)
        for h in range(hkv):
            k, v = OA.sequence_kv(pool_np, tables[b], n, h, ocfg, 0)
            want[b, h * g:(h + 1) * g] = OA.softmax_attend(qf[b, h * g:(h + 1) * g], k[keep], v[keep],
                                                           1.0 / math.sqrt(q.shape[2]))
    err = per_head_rel_l2(got, want)
    announce(f"  rel L2 {err:.2e}")
    assert err <= ATTN_RTOL
