"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: the same seeded workload build (all sequences appended through the
library), the same prepared step (quantize-append of one new token per
sequence at its last position, then decode over every sequence), checked on
sampled whole sequences that the oracle encodes and attends to itself from
the captured K/V: every slot byte of the sampled sequences bit-exact, and
their attention outputs within 2e-3 relative L2 per query head."""

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


def _picks(w):
    """Sequences whose slots (all KV heads) and outputs are checked: at least
    about a million slots per workload where the batch allows, every head,
    every block offset, first and last sequence (and for the log-normal mix
    the longest and the shortest)."""
    lens = sequence_lengths(w)
    if w.name == "3bit_nc":
        # 130944 compressed tokens x 8 heads each: 4.2 M slots, first and last included
        return (0, 2, 5, w.batch - 1)
    if w.lognormal_lengths:
        order = [int(i) for i in np.argsort(lens)[::-1]]
        return tuple(order[:10]) + (order[-1],)  # the ten longest and the shortest
    if w.batch <= 16:
        return tuple(range(w.batch))
    return tuple(sorted({0, w.batch // 3, 2 * w.batch // 3, w.batch - 1}))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "k8v4", "4bit_nc", "3bit_nc", "k3v4_nc", "k3v2_nc"])
def test_full_size_sampled_sequences(name):
    w = WORKLOADS[name]
    picks = _picks(w)
    announce(f"full-size {name}: sequences {picks}")
    built = WG.build(w, "cuda", n_pools=1, capture=picks)
    steps = WG.prepare_steps(built)
    qc, dc = steps[0]
    qc()
    dc()
    torch.cuda.synchronize()
    got_all = dc.out.cpu().numpy()
    ocfg = oracle_cfg(built.cfg)
    bs = w.block_size
    step_k = built.step_k.float().cpu().numpy()
    step_v = built.step_v.float().cpu().numpy()
    for b in picks:
        k, v = built.captured[b]
        n = k.shape[0]
        k = k.copy()
        v = v.copy()
        if n > 0:
            # the step appended its token at the last position
            k[n - 1] = step_k[b]
            v[n - 1] = step_v[b]
        nblk = max(1, -(-n // bs))
        pool = np.zeros((nblk, w.num_kv_heads, bs, ocfg.slot_size_aligned), np.uint8)
        for s0 in range(0, n, 16384):
            s1 = min(n, s0 + 16384)
            OX.append(pool, k[s0:s1], v[s0:s1], np.arange(s0, s1), ocfg, 0)
        # slot bytes of the whole sequence, read back through its block table
        if n > 0:
            pos = torch.arange(n, device="cuda")
            phys = built.tables[b, pos // bs].long()
            gpu_bytes = built.pools[0][phys, :, pos % bs, :].cpu().numpy()          # [n, Hkv, S]
            pos_np = np.arange(n)
            want_bytes = pool[pos_np // bs, :, pos_np % bs, :]
            mism = int((gpu_bytes != want_bytes).any(axis=-1).sum())
            announce(f"  seq {b}: {n} tokens, slots differing: {mism}")
            assert mism == 0
        ring = {}
        if w.ring:
            ring = dict(ring_k=built.ring_k[b:b + 1].float().cpu().numpy(),
                        ring_v=built.ring_v[b:b + 1].float().cpu().numpy(),
                        ring_lens=built.ring_lens[b:b + 1].cpu().numpy())
        q = built.q[b:b + 1].float().cpu().numpy()
        want = OA.decode_attention(q, pool, np.arange(nblk, dtype=np.int32)[None], [n], ocfg, 0, **ring)
        err = per_head_rel_l2(got_all[b:b + 1], want)
        announce(f"  seq {b}: attention rel L2 {err:.2e}")
        assert err <= ATTN_RTOL, err
