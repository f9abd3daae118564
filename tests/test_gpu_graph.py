"""Decode attention captured in a HIP graph and replayed.

The library allocates nothing and records no memset, so a caller can
capture a decode call (torch's graph capture: the call is issued on the
capturing stream) and replay it. Both decode entry points are captured: the
one with a caller workspace and the no-allocation one (its static scratch).
Between replays the inputs change in place with ordinary eager work (new
queries, shorter device-side lengths) and the stream synchronises; every
replay must equal, bit for bit, an eager call on the same inputs, and the
first is also checked against the oracle."""

import numpy as np
import pytest

from tests.gpu_common import ATTN_RTOL, announce, per_head_rel_l2
from tests.test_gpu_decode import _scenario

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("compressed_decode_attention_quantize_amd")

from oracle import attention as OA  # noqa: E402


@pytest.mark.parametrize("entry", ["workspace", "no_alloc"])
def test_decode_graph_replays_match_eager(entry):
    announce(f"decode graph capture, {entry} entry")
    lens = [1500, 260, 33]
    cfg, ocfg, pool_np, tables, q, ring = _scenario(128, 3, 3, True, 32, 8, lens, [128, 40, 0], 128, seed=91)
    pool = torch.from_numpy(pool_np).cuda()
    td = torch.from_numpy(tables).cuda()
    ld = torch.tensor(lens, dtype=torch.int32).cuda()
    rk, rv, rl = ring[0].cuda(), ring[1].cuda(), torch.from_numpy(ring[2]).cuda()
    qd = q.cuda()
    max_len = max(lens)
    kw = dict(ring_k=rk, ring_v=rv, ring_lens=rl)

    need, _ = tq.decode_workspace_size(cfg, len(lens), q.shape[1], max_len, rk.shape[2], 0)
    out_g = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws_g = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def call():
        if entry == "workspace":
            tq.decode_attention(cfg, 0, qd, pool, td, ld, max_len, out=out_g, workspace=ws_g, **kw)
        else:
            tq.decode_attention_no_alloc(cfg, 0, qd, pool, td, ld, max_len, out_g, **kw)

    # eager first: fills the library's per-device caches (resident
    # workgroups, the scratch address) outside the capture
    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    rng = np.random.default_rng(92)
    for rep in range(3):
        # eager work between replays: new queries, and from the second
        # replay on shorter device-side lengths (within max_len)
        q_new = torch.from_numpy(rng.standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16)
        qd.copy_(q_new.cuda())
        cur = list(lens) if rep == 0 else [max(0, n - 97 * rep) for n in lens]
        ld.copy_(torch.tensor(cur, dtype=torch.int32).cuda())
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out_g.cpu().numpy().copy()
        ref = tq.decode_attention(cfg, 0, qd, pool, td, ld, max_len, **kw)
        torch.cuda.synchronize()
        ref = ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"replay {rep} differs from the eager call"
        if rep == 0:
            want = OA.decode_attention(q_new.float().numpy(), pool_np, tables, cur, ocfg, 0,
                                       ring_k=ring[0].float().numpy(), ring_v=ring[1].float().numpy(),
                                       ring_lens=ring[2])
            err = per_head_rel_l2(got, want)
            announce(f"  replay 0 rel L2 {err:.2e}")
            assert err <= ATTN_RTOL
        announce(f"  replay {rep} (lengths {cur}) bit-identical to the eager call")
