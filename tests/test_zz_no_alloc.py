"""tq_decode_attention_no_alloc: the decode without a workspace argument
(the library's per-device static scratch instead), against
tq_decode_attention on the same inputs, through the C-ABI.

Two calls in a row, the second with a smaller input (the scratch then holds
the first call's partials), each bit-identical to tq_decode_attention's
output (same kernels, same launch) and within 2e-3 relative L2 per query
head of the oracle; a call whose partials do not fit is refused before
anything is enqueued."""

import ctypes

import numpy as np
import pytest

from tests.gpu_common import ATTN_RTOL, announce, per_head_rel_l2
from tests.test_gpu_decode import _scenario

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")

from oracle import attention as OA  # noqa: E402


def _both(cfg, ocfg, pool_np, tables, lens, q, ring, split):
    pool = torch.from_numpy(pool_np).cuda()
    kw = {}
    if ring is not None:
        kw = dict(ring_k=ring[0].cuda(), ring_v=ring[1].cuda(), ring_lens=torch.from_numpy(ring[2]).cuda())
    qd = q.cuda()
    td = torch.from_numpy(tables).cuda()
    ld = torch.tensor(lens, dtype=torch.int32).cuda()
    ref = tq.decode_attention(cfg, 0, qd, pool, td, ld, max(lens), split_tokens=split, **kw)
    out = torch.full_like(ref, float("nan"))
    tq.decode_attention_no_alloc(cfg, 0, qd, pool, td, ld, max(lens), out, split_tokens=split, **kw)
    torch.cuda.synchronize()
    want = OA.decode_attention(q.float().numpy(), pool_np, tables, lens, ocfg, 0,
                               ring_k=None if ring is None else ring[0].float().numpy(),
                               ring_v=None if ring is None else ring[1].float().numpy(),
                               ring_lens=None if ring is None else ring[2])
    return out.cpu().numpy(), ref.cpu().numpy(), want


@pytest.mark.parametrize("split", [0, 16])
def test_no_alloc_matches_workspace_entry_two_calls(split):
    # first call: 4-bit NC keys, G = 4, three sequences, a ring
    announce(f"no-alloc decode: large then small call, split={split}")
    lens1 = [2049, 300, 17]
    s1 = _scenario(128, 4, 4, True, 32, 8, lens1, [128, 40, 0], 128, seed=71)
    got, ref, want = _both(*s1[:4], lens1, s1[4], s1[5], split)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "first call differs from tq_decode_attention"
    err = per_head_rel_l2(got, want)
    announce(f"  first call rel L2 {err:.2e}")
    assert err <= ATTN_RTOL
    # second call, smaller: 3-bit NC keys at D = 96, one sequence, no ring
    lens2 = [200]
    s2 = _scenario(96, 3, 4, True, 16, 4, lens2, seed=72)
    got, ref, want = _both(*s2[:4], lens2, s2[4], s2[5], split)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "second call differs from tq_decode_attention"
    err = per_head_rel_l2(got, want)
    announce(f"  second call rel L2 {err:.2e}")
    assert err <= ATTN_RTOL


def test_no_alloc_refuses_what_does_not_fit():
    """8192 sequences x 128 query heads need far more partial rows than the
    32 MiB scratch holds: TQ_ERR_WORKSPACE, nothing launched (the device
    pointers below are never read)."""
    announce("no-alloc decode: oversized call refused")
    cfg = tq.config_from_preset("turboquant_4bit_nc", 128)
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    st = tq._lib.tq_decode_attention_no_alloc(ctypes.byref(cfg), 0, p, tq.BF16, 8192, 128, 8, p, 1, 16, p, 4096, p,
                                              65536, None, None, None, 0, 0.0, p, 0, None)
    assert st == 4, (st, tq.last_error())
    assert "scratch" in tq.last_error()
    torch.cuda.synchronize()
    assert int(buf.sum()) == 0
