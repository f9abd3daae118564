"""GPU parity: dequant reproduces the oracle's fp32 dequant bit for bit."""

import numpy as np
import pytest

from oracle import codec as OX
from tests.gpu_common import announce, oracle_cfg, oracle_pool

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")


@pytest.mark.parametrize("d,kb,vb,nc", [(64, 3, 4, False), (96, 3, 4, True), (128, 8, 4, False),
                                        (128, 4, 4, True), (128, 3, 3, True), (128, 4, 3, False),
                                        (96, 4, 3, True), (128, 3, 2, True), (96, 8, 2, False),
                                        (64, 4, 2, True)])
def test_dequant_bit_exact(d, kb, vb, nc):
    announce(f"dequant d={d} kb={kb} vb={vb} nc={nc}")
    cfg = tq.config_init(d, kb, vb, nc, 42)
    ocfg = oracle_cfg(cfg)
    hkv, n, nb = 2, 500, 40
    rng = np.random.default_rng(d + kb)
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = (rng.standard_normal((n, hkv, d)) * 3).astype(np.float32)
    mapping = rng.permutation(nb * 16)[:n]
    # the pool the oracle encodes is uploaded, so this checks dequant alone
    pool_np = oracle_pool(ocfg, 2, k, v, mapping, nb, hkv, 16)
    pool = torch.from_numpy(pool_np).cuda()
    ids = np.concatenate([mapping[:300], [-1, nb * 16, 5]]).astype(np.int64)
    kd, vd = tq.dequant(cfg, 2, pool, torch.from_numpy(ids).cuda())
    kd, vd = kd.cpu().numpy(), vd.cpu().numpy()
    for h in range(hkv):
        slots = OX.gather_slots(pool_np, mapping[:300], h)
        wk, wv = OX.dequant_f32(slots, ocfg, 2)
        assert np.array_equal(kd[:300, h].view(np.uint32), wk.view(np.uint32))
        assert np.array_equal(vd[:300, h].view(np.uint32), wv.view(np.uint32))
    assert (kd[300:302] == 0).all() and (vd[300:302] == 0).all()
    slot5 = OX.gather_slots(pool_np, [5], 0)
    wk5, _ = OX.dequant_f32(slot5, ocfg, 2)
    assert np.array_equal(kd[302, 0], wk5[0])
