"""GPU parity: quantize-and-append pool bytes equal the oracle's bit for bit."""

import math

import numpy as np
import pytest

from oracle import codec as OX
from tests.gpu_common import announce, oracle_cfg, oracle_pool

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _inputs(n, hkv, d, seed, dtype):
    """fp32 K/V with the awkward cases mixed in, rounded to the input dtype."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    k[:, :, rng.choice(d, 4, replace=False)] *= 10.0
    v[:, :, rng.choice(d, 4, replace=False)] *= 10.0
    k[3] = 0.0                              # zero key vectors
    v[4] = 0.25                             # constant value vectors
    k[5] *= 1e-3
    v[6] *= 300.0
    k[7] = rng.standard_normal((hkv, d)) * 1e-4
    v[8, :, :] = np.arange(d) % 16          # integer ramp
    # non-finite elements: a NaN, +inf and -inf in a key row each, then in a
    # value row each (index 0 for NaN coordinates; min/max skip NaN)
    k[11, :, 5] = np.nan
    k[12, :, 7] = np.inf
    k[13, :, 3] = -np.inf
    v[14, :, 2] = np.nan
    v[15, :, 1] = np.inf
    v[16, :, 0] = -np.inf
    # a signalling NaN (f32 inputs keep its bits): min/max skip it like a
    # quiet NaN, and its code is 0
    v.view(np.uint32)[17, :, 4] = 0x7F800001
    k.view(np.uint32)[18, :, 6] = 0x7F800001   # and in a key row (MSE: like a NaN; FP8: NaN code)
    tk = torch.from_numpy(k).to(DT[dtype])
    tv = torch.from_numpy(v).to(DT[dtype])
    if dtype != "f32":
        # the 16-bit formats' own signalling-NaN pattern (the conversion above
        # quiets the f32 one)
        tv.view(torch.int16)[17, :, 4] = 0x7F81 if dtype == "bf16" else 0x7C01
        tk.view(torch.int16)[18, :, 6] = 0x7F81 if dtype == "bf16" else 0x7C01
    return tk, tv, tk.float().numpy(), tv.float().numpy()


CASES = [
    # (head_dim, key_bits, value_bits, nc)
    (64, 3, 4, False), (64, 4, 3, False), (64, 8, 4, False),
    (96, 3, 4, True), (96, 4, 4, False), (96, 8, 3, False),
    (128, 8, 4, False), (128, 4, 4, True), (128, 3, 3, True), (128, 3, 4, True), (128, 4, 3, False),
    # 2-bit values
    (64, 8, 2, False), (96, 3, 2, True), (128, 3, 2, True), (128, 4, 2, False),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("d,kb,vb,nc", CASES)
def test_pool_bytes_bit_exact(d, kb, vb, nc, dtype):
    announce(f"quantize d={d} kb={kb} vb={vb} nc={nc} dtype={dtype}")
    cfg = tq.config_init(d, kb, vb, nc, 42)
    ocfg = oracle_cfg(cfg)
    n, hkv, bs, nb = 1037, 3, 16, 80
    tk, tv, k, v = _inputs(n, hkv, d, seed=d * 100 + kb * 10 + vb, dtype=dtype)
    rng = np.random.default_rng(5)
    mapping = rng.permutation(nb * bs)[:n].astype(np.int64)
    mapping[::97] = -1                              # skipped tokens
    mapping[10] = nb * bs + 5                       # out of range: skipped too
    pool = torch.zeros((nb, hkv, bs, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    tq.quantize_append(cfg, 3, tk.cuda(), tv.cuda(), torch.from_numpy(mapping).cuda(), pool)
    got = pool.cpu().numpy()
    want_map = mapping.copy()
    want_map[10] = -1
    want = oracle_pool(ocfg, 3, k, v, want_map, nb, hkv, bs)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} bytes differ; first at {mism[:5].tolist()}"


@pytest.mark.parametrize("d,kb", [(128, 4), (128, 3), (96, 4), (96, 3), (64, 4), (64, 3)])
def test_keys_on_midpoint_ties_bit_exact(d, kb):
    """Keys whose rotated coordinates fall exactly on each Lloyd-Max midpoint
    and one ulp either side (fp32 inputs, so the kernel sees the same
    coordinates): pool bytes equal the oracle's, and the codes at the tied
    coordinates are the number of midpoints strictly below."""
    from tests.midpoint_keys import tie_keys
    announce(f"quantize midpoint ties d={d} kb={kb}")
    cfg = tq.config_init(d, kb, 4, False, 42)
    ocfg = oracle_cfg(cfg)
    keys, cases = tie_keys(ocfg, layer_idx=2, seed=d + kb)
    n, bs = len(keys), 16
    nb = (n + bs - 1) // bs
    rng = np.random.default_rng(d * 10 + kb)
    k = keys[:, None, :].copy()
    v = rng.standard_normal((n, 1, d)).astype(np.float32)
    mapping = np.arange(n, dtype=np.int64)
    pool = torch.zeros((nb, 1, bs, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    tq.quantize_append(cfg, 2, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                       torch.from_numpy(mapping).cuda(), pool)
    got = pool.cpu().numpy()
    want = oracle_pool(ocfg, 2, k, v, mapping, nb, 1, bs)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} bytes differ; first at {mism[:5].tolist()}"
    idx = OX.decode_slot_fields(got.reshape(-1, cfg.slot_size_aligned)[:n], ocfg)["idx"]
    for row, i, kk, off in cases:
        assert idx[row, i] == (kk + 1 if off > 0 else kk), (row, i, kk, off)


def test_tiny_workload_prefill_then_decode_append():
    """511 tokens appended in bulk, then one more (the tiny workload)."""
    from workloads import tiny_numpy
    announce("quantize tiny workload")
    k, v, _ = tiny_numpy()
    cfg = tq.config_init(64, 3, 4, False, 42)
    ocfg = oracle_cfg(cfg)
    pool = torch.zeros((32, 2, 16, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    ids = torch.arange(512, dtype=torch.int64, device="cuda")
    tq.quantize_append(cfg, 0, torch.from_numpy(k[:511]).cuda(), torch.from_numpy(v[:511]).cuda(), ids[:511], pool)
    tq.quantize_append(cfg, 0, torch.from_numpy(k[511:]).cuda(), torch.from_numpy(v[511:]).cuda(), ids[511:], pool)
    want = oracle_pool(ocfg, 0, k, v, np.arange(512), 32, 2, 16)
    assert np.array_equal(pool.cpu().numpy(), want)


def test_fp8_keys_every_bf16_pattern():
    """All 65536 bf16 bit patterns (NaN, inf, subnormals, saturation) as keys."""
    announce("quantize fp8 exhaustive")
    cfg = tq.config_from_preset("turboquant_k8v4", 128)
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    k = bits.reshape(512, 1, 128)
    v = torch.zeros_like(k)
    pool = torch.zeros((32, 1, 16, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    tq.quantize_append(cfg, 0, k.cuda(), v.cuda(), torch.arange(512, dtype=torch.int64, device="cuda"), pool)
    got = pool.cpu().numpy().reshape(512, cfg.slot_size_aligned)[:, :128].reshape(-1)
    want = OX.fp8_e4m3fn_encode(k.float().numpy().reshape(-1))
    assert np.array_equal(got, want)


def test_layers_use_their_own_signs():
    announce("quantize layer seeds")
    cfg = tq.config_from_preset("turboquant_4bit_nc", 128)
    ocfg = oracle_cfg(cfg)
    tk, tv, k, v = _inputs(64, 2, 128, seed=9, dtype="bf16")
    for layer in (0, 5):
        pool = torch.zeros((4, 2, 16, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
        tq.quantize_append(cfg, layer, tk.cuda(), tv.cuda(), torch.arange(64, dtype=torch.int64, device="cuda"), pool)
        want = oracle_pool(ocfg, layer, k, v, np.arange(64), 4, 2, 16)
        assert np.array_equal(pool.cpu().numpy(), want)


def test_strided_rows_and_block_size_32():
    """K/V as views into a wider [T, 2*Hkv*D] buffer (token stride > row)."""
    announce("quantize strided rows bs=32")
    cfg = tq.config_from_preset("turboquant_k3v4_nc", 96)
    ocfg = oracle_cfg(cfg)
    hkv, n = 4, 300
    rng = np.random.default_rng(11)
    both = rng.standard_normal((n, 2, hkv, 96)).astype(np.float32)
    t = torch.from_numpy(both).to(torch.bfloat16).cuda()
    k, v = t[:, 0], t[:, 1]
    assert k.stride(0) == 2 * hkv * 96
    pool = torch.zeros((12, hkv, 32, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    mapping = np.random.default_rng(12).permutation(12 * 32)[:n]
    tq.quantize_append(cfg, 1, k, v, torch.from_numpy(mapping).cuda(), pool)
    kk = t.float().cpu().numpy()
    want = oracle_pool(ocfg, 1, kk[:, 0], kk[:, 1], mapping, 12, hkv, 32)
    assert np.array_equal(pool.cpu().numpy(), want)


@pytest.mark.parametrize("bs", [7, 24])
def test_block_size_not_power_of_two(bs):
    """Slot -> (block, offset) by division rather than shift and mask."""
    announce(f"quantize block size {bs}")
    cfg = tq.config_from_preset("turboquant_4bit_nc", 128)
    ocfg = oracle_cfg(cfg)
    hkv, n, nb = 3, 200, 40
    rng = np.random.default_rng(bs)
    k = rng.standard_normal((n, hkv, 128)).astype(np.float32)
    v = rng.standard_normal((n, hkv, 128)).astype(np.float32)
    mapping = rng.permutation(nb * bs)[:n].astype(np.int64)
    pool = torch.zeros((nb, hkv, bs, cfg.slot_size_aligned), dtype=torch.uint8, device="cuda")
    tq.quantize_append(cfg, 2, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                       torch.from_numpy(mapping).cuda(), pool)
    want = oracle_pool(ocfg, 2, k, v, mapping, nb, hkv, bs)
    assert np.array_equal(pool.cpu().numpy(), want)


def test_empty_append_is_noop():
    cfg = tq.config_from_preset("turboquant_3bit_nc", 128)
    pool = torch.full((2, 1, 16, cfg.slot_size_aligned), 7, dtype=torch.uint8, device="cuda")
    e = torch.empty((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    tq.quantize_append(cfg, 0, e, e, torch.empty((0,), dtype=torch.int64, device="cuda"), pool)
    assert (pool == 7).all()
