"""GPU parity of the overlapped write path of the k3v4_nc workload: a
65536-token prefill quantize-append on a second stream while decode attention
runs on the main stream over the same paged pool (disjoint slots), in the
launch configuration bench.py times.

Write path after the hnwysp.cn article on the stand-alone turboquant project,
write-path section (writes land chunk-wise, off the per-token hot path); the
workload is D = 96, 16 q / 4 KV heads, 64 log-normal sequences in one shared
pool plus the prefill of a 65th sequence into spare blocks.

Checked:
  * the prefill's slots bit-exact against the oracle's append of the same K/V;
  * every other pool byte unchanged by the overlapped pair;
  * the decode output identical to the same decode run alone, and within
    2e-3 relative L2 per query head of the oracle on the longest and the
    shortest sequence.
"""

import numpy as np
import pytest

from oracle import attention as OA
from oracle import codec as OX
from tests.gpu_common import ATTN_RTOL, announce, oracle_cfg, per_head_rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")

from workloads import WORKLOADS, sequence_lengths  # noqa: E402
from workloads import gpu as WG  # noqa: E402


@pytest.mark.timeout(600)
def test_prefill_on_second_stream_during_decode():
    w = WORKLOADS["k3v4_nc"]
    lens = sequence_lengths(w)
    picks = (int(np.argmax(lens)), int(np.argmin(lens)))
    n = w.prefill_tokens
    spare_blocks = -(-n // w.block_size)
    announce(f"overlap k3v4_nc: prefill {n} tokens on a side stream, decode sequences {picks}")
    built = WG.build(w, "cuda", n_pools=1, capture=picks, extra_blocks=spare_blocks)
    pool = built.pools[0]
    dc = WG.prepare_steps(built)[0][1]
    k, v = WG.prefill_source(w, "cuda").kv(n)
    ids_np = WG.spare_slot_ids(built, n)
    ids = torch.from_numpy(ids_np).cuda()
    side = torch.cuda.Stream()
    pre = tq.prepare_quantize(built.cfg, 0, k, v, ids, pool, stream=side.cuda_stream)
    main = torch.cuda.current_stream()

    # the decode alone, and the pool before the pair
    dc()
    torch.cuda.synchronize()
    solo = dc.out.clone()
    before = pool.clone()
    dc.out.fill_(float("nan"))

    # the pair: prefill enqueued first on the side stream, decode on the main one
    side.wait_stream(main)
    pre()
    dc()
    main.wait_stream(side)
    torch.cuda.synchronize()

    # decode: identical to the solo run (the prefill writes slots it never reads)
    assert torch.equal(dc.out, solo), "overlapped decode differs from the decode alone"

    # untouched bytes: every block outside the prefill's
    written = np.unique(ids_np // w.block_size)
    keep = torch.ones(pool.shape[0], dtype=torch.bool, device="cuda")
    keep[torch.from_numpy(written).cuda()] = False
    assert torch.equal(pool[keep], before[keep]), "the prefill changed slots outside its blocks"

    # the prefill's slots against the oracle's append
    ocfg = oracle_cfg(built.cfg)
    kk = k.float().cpu().numpy()
    vv = v.float().cpu().numpy()
    got = pool[torch.from_numpy(written).cuda()].cpu().numpy()          # [nw, Hkv, bs, S]
    want = np.zeros_like(got)
    remap = {int(blk): i for i, blk in enumerate(written)}
    local_ids = np.array([remap[int(s // w.block_size)] * w.block_size + int(s % w.block_size) for s in ids_np])
    for s0 in range(0, n, 16384):
        s1 = min(n, s0 + 16384)
        OX.append(want, kk[s0:s1], vv[s0:s1], local_ids[s0:s1], ocfg, 0)
    mism = int((got != want).any(axis=-1).sum())
    announce(f"  prefill slots differing: {mism}")
    assert mism == 0

    # decode against the oracle on the sampled sequences
    out = dc.out.cpu().numpy()
    bs = w.block_size
    for b in picks:
        kc, vc = built.captured[b]
        m = kc.shape[0]
        nblk = max(1, -(-m // bs))
        opool = np.zeros((nblk, w.num_kv_heads, bs, ocfg.slot_size_aligned), np.uint8)
        for s0 in range(0, m, 16384):
            s1 = min(m, s0 + 16384)
            OX.append(opool, kc[s0:s1], vc[s0:s1], np.arange(s0, s1), ocfg, 0)
        q = built.q[b:b + 1].float().cpu().numpy()
        ref = OA.decode_attention(q, opool, np.arange(nblk, dtype=np.int32)[None], [m], ocfg, 0)
        err = per_head_rel_l2(out[b:b + 1], ref)
        announce(f"  seq {b} ({m} tokens): attention rel L2 {err:.2e}")
        assert err <= ATTN_RTOL, err
