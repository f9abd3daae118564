"""Benchmark of the TurboQuant decode hot path on one MI355X.

A step is one pass of the whole path over one batch: quantize-append one new
token per sequence into the paged pool, then fused decode attention over
every sequence's full context. Inputs are seeded synthetic data already
resident in HBM (see workloads/). Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4bit_nc]

Timing, after 0.25 s of back-to-back decode launches (clock ramp) and W
warm-up steps, in this order:
  1. K steps with HIP events around every quantize and decode launch
     (per-call durations, reported under decode.ms_mean/p10/p50/p90 and
     quantize_step; event records cost the stream a few microseconds each);
  2. K decode launches back to back between two HIP events: the sustained
     per-launch duration of the decode call (split + reduce kernels), the
     "dominant kernel" time of the roofline object;
  3. the timed region: exactly K steps back to back, bracketed by
     synchronisation, with nothing inside the loop but the two calls; it
     gives `value` and `ms_per_step`.
Pools too small to defeat the 256 MB Infinity Cache are replicated and
rotated (step i reads pool i mod n).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 << 20         # Infinity Cache
PMC_FILE = os.path.join(ROOT, "profiles", "decode_pmc.json")


def _sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_sha():
    """Hash of the sources that decide a decode launch's traffic: the
    kernels and the host-side work plan (range lengths, partial slots)."""
    c = os.path.join(ROOT, "compressed_decode_attention_quantize_amd", "csrc")
    return _sha([os.path.join(c, f) for f in ("tq_decode.hip", "tq_mfma.h", "tq_device.h", "tq_host.cpp", "tq_internal.h")])


def _traffic(workload_name, per_launch_bytes):
    """HBM bytes per decode launch from committed PMC counters, if they were
    taken on the current kernel source; else None."""
    try:
        with open(PMC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload_name)
    if not entry or entry.get("source_sha") != kernel_source_sha():
        return None
    return entry.get("traffic_bytes_per_launch")


def host_description():
    """The host CPU as the oracle baseline ran on it: model name, the
    machine's logical CPU count, and the CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable}


# Worker processes of the all-cores oracle baseline: at most this many (the
# host share of one GPU), each single-threaded.
CPU_WORKERS_MAX = 16


def _oracle_decode_worker(job):
    """One single-threaded worker of the all-cores baseline: the oracle's
    decode of the sample sequence, repeated until `budget_s` has passed.
    Returns (KV tokens attended, seconds)."""
    q, pool, table, n, ring, cfg_fields, budget_s, start_at = job
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    from oracle import config as OC

    ocfg = OC.TQConfig(**cfg_fields)
    tokens = 0
    with threadpool_limits(limits=1):
        while time.time() < start_at:       # all workers start together
            time.sleep(0.001)
        t0 = time.perf_counter()
        while True:
            OA.decode_attention(q, pool, table, [n], ocfg, 0, **ring)
            tokens += n + (int(ring["ring_lens"][0]) if ring else 0)
            el = time.perf_counter() - t0
            if el >= budget_s:
                return tokens, el


def cpu_baseline(built, budget_s: float):
    """The oracle's decode attention timed on host cores over a bounded
    sample (one whole sequence of the same workload, oracle-encoded from the
    same K/V), in KV tokens per second: (i) one core, one process; (ii) all
    usable cores (at most CPU_WORKERS_MAX), one single-threaded worker process
    per core, each decoding the sample sequence repeatedly. The decode cost
    is the same for every sequence of a uniform workload, so (ii) is the
    throughput of sharding the batch by sequence."""
    import multiprocessing as mp

    from oracle import codec as OX
    from oracle import config as OC

    w = built.w
    cfg = built.cfg
    cfg_fields = dict(head_dim=cfg.head_dim, key_quant_bits=cfg.key_quant_bits,
                      value_quant_bits=cfg.value_quant_bits, seed=int(cfg.seed),
                      norm_correction=bool(cfg.norm_correction))
    ocfg = OC.TQConfig(**cfg_fields)
    b = min(built.captured)
    k, v = built.captured[b]
    n = k.shape[0]
    bs = w.block_size
    nblk = max(1, -(-n // bs))
    pool = np.zeros((nblk, w.num_kv_heads, bs, ocfg.slot_size_aligned), np.uint8)
    for s0 in range(0, n, 16384):
        OX.append(pool, k[s0:s0 + 16384], v[s0:s0 + 16384], np.arange(s0, min(n, s0 + 16384)), ocfg, 0)
    q = built.q[b:b + 1].float().cpu().numpy()
    table = np.arange(nblk, dtype=np.int32)[None]
    ring = {}
    if w.ring:
        ring = dict(ring_k=built.ring_k[b:b + 1].float().cpu().numpy(),
                    ring_v=built.ring_v[b:b + 1].float().cpu().numpy(),
                    ring_lens=np.array([w.ring]))
    host = host_description()
    # (i) one core, in this process
    tok1, el1 = _oracle_decode_worker((q, pool, table, n, ring, cfg_fields, budget_s, 0.0))
    # (ii) all cores: fresh interpreters (spawn), none of which touches the GPU
    nw = max(1, min(CPU_WORKERS_MAX, host["usable_cpus"]))
    ctx = mp.get_context("spawn")
    with ctx.Pool(nw) as pool_:
        start_at = time.time() + 5.0 + 0.1 * nw    # after every worker has imported numpy
        res = pool_.map(_oracle_decode_worker,
                        [(q, pool, table, n, ring, cfg_fields, budget_s, start_at)] * nw, chunksize=1)
    tok_all = sum(t for t, _ in res)
    el_all = max(e for _, e in res)
    seq = f"sequence {b} ({n} compressed + {w.ring} ring tokens, {w.num_q_heads} q heads)"
    return {"value": tok1 / el1, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{seq} decoded {tok1 // max(n + w.ring, 1)}x in {el1:.1f} s, numpy single-threaded",
            "all_cores": {"value": tok_all / el_all, "unit": "KV tokens/s", "cores": nw,
                          "sample": f"{seq} decoded {tok_all // max(n + w.ring, 1)}x by {nw} single-threaded "
                                    f"worker processes over {el_all:.1f} s"},
            "host": host}


def bulk_quantize(built, tq, torch, chunk=65536, reps=5):
    """Quantize-append throughput: `chunk`-token appends into pool 0 (rewriting
    the leading positions of sequences 0, 1, ... until `chunk` tokens, or all
    of them), events around each call."""
    from workloads import KVSource, slot_ids_for
    w = built.w
    parts, n = [], 0
    for b in range(len(built.lens_np)):
        take = min(chunk - n, int(built.lens_np[b]))
        if take > 0:
            parts.append(slot_ids_for(built.tables_np, b, 0, take, w.block_size))
            n += take
        if n == chunk:
            break
    src = KVSource(w, "cuda", stream_id=77)
    k, v = src.kv(n)
    ids = torch.from_numpy(np.concatenate(parts)).cuda()
    call = tq.prepare_quantize(built.cfg, 0, k, v, ids, built.pools[0])
    for _ in range(2):
        call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    return n, ms


def copy_probe(torch, nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of ``nbytes`` (torch copy_ of a float32
    buffer): the measured copy bandwidth (read + write bytes / time), and the
    reference kernel the PMC byte counters are scaled against."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms, "GBps": 2 * nbytes / (ms / 1e3) / 1e9}


def clock_warmup(torch, calls, seconds: float = 0.25):
    """Back-to-back launches for `seconds` before anything is measured: the
    GPU ramps its clocks up over tens of milliseconds of load, and a serving
    loop runs at the ramped clocks."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            calls[i % len(calls)]()
            i += 1
        torch.cuda.synchronize()


def _timed(torch, fn, reps):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def ring_flush(built, tq, torch, reps=10):
    """One ring flush: every sequence's 128 ring tokens quantize-appended as a
    chunk (one call, batch x ring tokens) into spare blocks of pool 0."""
    from workloads import KVSource
    from workloads import gpu as WG
    w = built.w
    n = w.batch * w.ring
    k, v = KVSource(w, "cuda", stream_id=78).kv(n)
    ids = torch.from_numpy(WG.spare_slot_ids(built, n)).cuda()
    call = tq.prepare_quantize(built.cfg, 0, k, v, ids, built.pools[0])
    call()
    ms = _timed(torch, call, reps)
    qbpt = WG.quantize_bytes_per_token(built)
    return {"tokens": n, "ms": ms, "tokens_per_s": n / (ms / 1e3), "GBps": n * qbpt / (ms / 1e3) / 1e9}


def ring_step(built, tq, torch, reps=10):
    """The device-side ring manager on full rings: tq_ring_flush (every
    sequence's 128 ring tokens compressed at its next positions, lengths
    advanced on the device) then tq_ring_append of one new token per sequence.
    Spare blocks extend each sequence's block table; the lengths and rings are
    restored between timed reps (outside the events)."""
    from workloads import KVSource
    w = built.w
    bs = w.block_size
    extra = -(-w.ring // bs)
    spare = np.asarray(built.spare_blocks, dtype=np.int32)
    assert len(spare) >= w.batch * extra, "not enough spare blocks"
    lens = built.lens_np.astype(np.int64)
    tables = np.zeros((w.batch, int((lens + w.ring + bs - 1).max() // bs)), np.int32)
    for b in range(w.batch):
        nb = -(-int(lens[b]) // bs)
        tables[b, :nb] = built.tables_np[b, :nb]
        tables[b, nb:nb + extra] = spare[b * extra:(b + 1) * extra]
    g_tab = torch.from_numpy(tables).cuda()
    sl0 = built.seq_lens.clone()
    rl0 = torch.full((w.batch,), w.ring, dtype=torch.int32, device="cuda")
    rk, rv = built.ring_k.clone(), built.ring_v.clone()
    sl, rl = sl0.clone(), rl0.clone()
    kn, vn = KVSource(w, "cuda", stream_id=77).kv(w.batch)
    kn = kn.reshape(w.batch, w.num_kv_heads, w.head_dim).contiguous()
    vn = vn.reshape(w.batch, w.num_kv_heads, w.head_dim).contiguous()
    times = []
    for i in range(reps + 2):
        sl.copy_(sl0)
        rl.copy_(rl0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        tq.ring_step(built.cfg, 0, kn, vn, rk, rv, rl, sl, g_tab, built.pools[0])
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1))
    assert rl.cpu().tolist() == [1] * w.batch and (sl - sl0).cpu().tolist() == [w.ring] * w.batch
    ms = float(np.mean(times))
    n = w.batch * w.ring
    return {"tokens_flushed": n, "ms": ms, "tokens_per_s": n / (ms / 1e3)}


def concurrent_prefill(built, tq, torch, steps, reps=10):
    """Decode on the current stream with a prefill quantize-append of
    ``prefill_tokens`` tokens (a sequence outside the batch, written to spare
    blocks) on a second stream: each alone, then both together."""
    from workloads import gpu as WG
    w = built.w
    n = w.prefill_tokens
    k, v = WG.prefill_source(w, "cuda").kv(n)
    ids = torch.from_numpy(WG.spare_slot_ids(built, n)).cuda()
    side = torch.cuda.Stream()
    pre = tq.prepare_quantize(built.cfg, 0, k, v, ids, built.pools[0], stream=side.cuda_stream)
    main = torch.cuda.current_stream()
    dec = steps[0][1]

    def prefill_alone():
        side.wait_stream(main)
        pre()
        main.wait_stream(side)

    def both():
        side.wait_stream(main)
        pre()
        dec()
        main.wait_stream(side)

    prefill_alone()
    both()
    pre_ms = _timed(torch, prefill_alone, reps)
    dec_ms = _timed(torch, dec, reps)
    both_ms = _timed(torch, both, reps)
    pbytes = n * WG.quantize_bytes_per_token(built)
    dbytes = WG.decode_bytes(built)
    return {"prefill_tokens": n, "prefill_ms": pre_ms, "prefill_tokens_per_s": n / (pre_ms / 1e3),
            "prefill_GBps": pbytes / (pre_ms / 1e3) / 1e9, "decode_ms": dec_ms, "overlapped_ms": both_ms,
            "overlapped_GBps": (pbytes + dbytes) / (both_ms / 1e3) / 1e9}


# The pages' own figures for the four presets (vLLM API page
# "vllm.model_executor.layers.quantization.turboquant", TurboQuantConfig
# docstring, named presets): KV compression and perplexity change, as quoted
# (model and data unnamed). Context for the measurements, not a target.
PAGE_PRESET_FIGURES = {
    "turboquant_k8v4": {"compression_quoted": "2.6x", "ppl_delta_quoted": "+1.17%"},
    "turboquant_4bit_nc": {"compression_quoted": "3.8x", "ppl_delta_quoted": "+2.71%"},
    "turboquant_k3v4_nc": {"compression_quoted": "~3.5x", "ppl_delta_quoted": "+10.63%"},
    "turboquant_3bit_nc": {"compression_quoted": "4.9x", "ppl_delta_quoted": "+20.59%"},
}


def page_context(w, cfg):
    """The preset's quoted figures beside the ratio its slot size gives
    (bf16 K + V = 4 D bytes per token and head, over slot_size_aligned)."""
    out = {"slot_bytes": cfg.slot_size_aligned,
           "compression_vs_bf16_from_slot_size": round(4 * w.head_dim / cfg.slot_size_aligned, 3)}
    if w.preset in PAGE_PRESET_FIGURES:
        out.update(PAGE_PRESET_FIGURES[w.preset])
        out["source"] = "vLLM API page TurboQuantConfig docstring, named presets (model and data unnamed)"
    return out


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16/bf16 matrix peak, published


def prefill_flops(w, hist_lens, chunk) -> int:
    """Dense work of one continuation prefill: per (chunk token, query head),
    2 D flops for q.k and 2 D for p.v over every visible key (history plus
    the causal part of the chunk)."""
    total = 0
    for L in hist_lens:
        vis = chunk * int(L) + chunk * (chunk + 1) // 2
        total += 4 * w.head_dim * w.num_q_heads * vis
    return total


def prefill_cpu_baseline(built, chunk_q, chunk_k, chunk_v, budget_s: float):
    """The oracle's continuation prefill on host cores: sequence 0's history
    with the first rows of its chunk, repeated for about budget_s."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    from oracle import codec as OX
    from oracle import config as OC

    w, cfg = built.w, built.cfg
    ocfg = OC.TQConfig(head_dim=cfg.head_dim, key_quant_bits=cfg.key_quant_bits,
                       value_quant_bits=cfg.value_quant_bits, seed=int(cfg.seed),
                       norm_correction=bool(cfg.norm_correction))
    k, v = built.captured[0]
    n = k.shape[0]
    bs = w.block_size
    nblk = max(1, -(-n // bs))
    pool = np.zeros((nblk, w.num_kv_heads, bs, ocfg.slot_size_aligned), np.uint8)
    for s0 in range(0, n, 16384):
        OX.append(pool, k[s0:s0 + 16384], v[s0:s0 + 16384], np.arange(s0, min(n, s0 + 16384)), ocfg, 0)
    rows = 8
    q = chunk_q[:rows].float().cpu().numpy()
    kc = chunk_k[:rows].float().cpu().numpy()
    vc = chunk_v[:rows].float().cpu().numpy()
    table = np.arange(nblk, dtype=np.int32)[None]
    toks = reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            OA.prefill_attention(q, kc, vc, [0, rows], pool, table, [n], ocfg, 0)
            toks += rows
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return {"value": toks / el, "unit": "chunk tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"sequence 0: {rows} chunk rows over its {n}-token history, {w.num_q_heads} q heads, "
                      f"{reps}x in {el:.1f} s, numpy single-threaded"}


def run_prefill(args, w, tq, torch):
    """Continuation prefill step: attention of every sequence's new chunk to
    its compressed history and causally to itself, then quantize-append of the
    chunk (into spare blocks)."""
    from workloads import KVSource
    from workloads import gpu as WG

    spare = w.batch * -(-w.chunk // w.block_size)
    print(f"[bench] building {w.name}: {w.description}", file=sys.stderr, flush=True)
    built = WG.build(w, "cuda", n_pools=1, capture=(0,), extra_blocks=spare)
    n = w.batch * w.chunk
    src = KVSource(w, "cuda", stream_id=55)
    ck, cv = src.kv(n)                                   # [n, Hkv, D] bf16
    cq = KVSource(w, "cuda", stream_id=56).q(n)            # [n, Hq, D] bf16
    cu = torch.arange(0, n + 1, w.chunk, dtype=torch.int32, device="cuda")
    out = torch.empty((n, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    need = tq.prefill_workspace_size(built.cfg, w.batch, w.num_q_heads, w.num_kv_heads, w.chunk,
                                     built.max_seq_len, built.tables.shape[1], tq.BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ids = torch.from_numpy(WG.spare_slot_ids(built, n)).cuda()

    def attn():
        tq.prefill_attention(built.cfg, 0, cq, ck, cv, cu, w.chunk, built.pools[0], built.tables, built.seq_lens,
                             built.max_seq_len, out=out, workspace=ws)

    append = tq.prepare_quantize(built.cfg, 0, ck, cv, ids, built.pools[0])
    clock_warmup(torch, [attn])
    for _ in range(args.warmup):
        attn()
        append()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        ev[i][0].record()
        attn()
        ev[i][1].record()
        append()
        ev[i][2].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / K
    att_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    app_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    flops = prefill_flops(w, built.lens_np, w.chunk)
    tflops = flops / (float(att_ms.mean()) / 1e3) / 1e12
    result = {
        "metric": "continuation-prefill chunk tokens/s (attention to compressed history + chunk append)",
        "value": n / (ms_step / 1e3),
        "unit": "chunk tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "preset": w.preset,
                   "head_dim": w.head_dim, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "batch": w.batch, "history": int(built.max_seq_len), "chunk": w.chunk,
                   "block_size": w.block_size, "parallelism": "single GPU"},
        "prefill": {"ms_mean": float(att_ms.mean()), "ms_p50": float(np.median(att_ms)), "flops": flops,
                    "TFLOPs": tflops},
        "append": {"ms_mean": float(app_ms.mean()), "tokens": n},
        "roofline": {"bound": "mfma", "kernel": "tq_prefill_attention (attention + reduce kernels)",
                     "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None},
        "wall_s_timed": wall,
        "library": tq.version(),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = prefill_cpu_baseline(built, cq, ck, cv, args.cpu_budget)
    print(json.dumps(result))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="4bit_nc")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_decode_attention_quantize_amd as tq
    from workloads import WORKLOADS
    from workloads import gpu as WG

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = WORKLOADS[args.workload]
    if w.chunk:
        run_prefill(args, w, tq, torch)
        return
    cfg = tq.config_from_preset(w.preset, w.head_dim) if w.preset else \
        tq.config_init(w.head_dim, w.key_bits, w.value_bits, w.norm_correction, 42)
    from workloads import sequence_lengths
    pool_bytes = int(sequence_lengths(w).sum()) * w.num_kv_heads * cfg.slot_size_aligned
    n_pools = 1 if pool_bytes > 2 * MALL_BYTES else max(1, -(-3 * MALL_BYTES // max(pool_bytes, 1)))
    n_pools = min(n_pools, 8)
    print(f"[bench] building {w.name}: {w.description}; {n_pools} pool(s) of {pool_bytes / 1e6:.1f} MB",
          file=sys.stderr, flush=True)
    spare = (w.batch * -(-w.ring // w.block_size)) + -(-w.prefill_tokens // w.block_size)
    built = WG.build(w, "cuda", n_pools=n_pools, capture=(0,), extra_blocks=spare)
    steps = WG.prepare_steps(built, args.split_tokens)
    _, nsplit = tq.decode_workspace_size(cfg, w.batch, w.num_q_heads, built.max_seq_len, w.ring, args.split_tokens)

    clock_warmup(torch, [dc for _, dc in steps])
    for i in range(args.warmup):
        qc, dc = steps[i % n_pools]
        qc()
        dc()
    K = args.steps
    # Instrumented region: K steps with HIP events around every call on the
    # stream the kernels run on (per-call durations). Each event record costs
    # the stream a few microseconds, so these steps run slower than the timed
    # ones; the per-call durations include that.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        qc, dc = steps[i % n_pools]
        ev[i][0].record()
        qc()
        ev[i][1].record()
        dc()
        ev[i][2].record()
    torch.cuda.synchronize()
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    qnt_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    instr_ms_step = ev[0][0].elapsed_time(ev[-1][2]) / K
    # Decode launches back to back between two events on the same stream (the
    # pools rotate as in the steps): the sustained per-launch decode duration
    # that the roofline divides the algorithmic bytes by.
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record()
    for i in range(K):
        steps[i % n_pools][1]()
    d1.record()
    torch.cuda.synchronize()
    dec_b2b = d0.elapsed_time(d1) / K
    # Timed region, last (the GPU has reached its working clocks): exactly K
    # steps back to back, bracketed by synchronisation, no instrumentation
    # inside the loop.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        qc, dc = steps[i % n_pools]
        qc()
        dc()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K

    kv_tokens = int(built.lens_np.sum()) + w.batch * w.ring
    value = kv_tokens / (ms_step / 1e3)
    dbytes = WG.decode_bytes(built)
    dec_mean = float(dec_ms.mean())
    achieved = dbytes / (dec_b2b / 1e3) / 1e9
    traffic = _traffic(w.name, dbytes)

    nq, qms = bulk_quantize(built, tq, torch)
    qbpt = WG.quantize_bytes_per_token(built)
    extra = {}
    if w.ring:
        extra["ring_flush"] = ring_flush(built, tq, torch)
        extra["ring_step"] = ring_step(built, tq, torch)
    if w.prefill_tokens:
        extra["concurrent_prefill"] = concurrent_prefill(built, tq, torch, steps)
    extra["copy_probe"] = copy = copy_probe(torch)

    result = {
        "metric": "decode-attn KV tokens/s + achieved HBM GB/s (% peak); quantize tokens/s",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "preset": w.preset,
                   "head_dim": w.head_dim, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "batch": w.batch, "context": w.context, "ring": w.ring, "block_size": w.block_size,
                   "kv_tokens_per_step": kv_tokens, "splits_per_seq": nsplit, "pools_rotated": n_pools,
                   "parallelism": "single GPU"},
        "decode": {"ms_back_to_back": dec_b2b,
                   "ms_mean": dec_mean, "ms_p10": float(np.percentile(dec_ms, 10)),
                   "ms_p50": float(np.median(dec_ms)), "ms_p90": float(np.percentile(dec_ms, 90)),
                   "algorithmic_bytes": dbytes, "GBps": achieved, "pct_hbm_peak": 100 * achieved / HBM_PEAK_GBS,
                   "kv_tokens_per_s": kv_tokens / (dec_b2b / 1e3)},
        "quantize_step": {"ms_mean": float(qnt_ms.mean()), "tokens": w.batch},
        "timing": {"value": "K steps back to back, bracketed by synchronisation",
                   "roofline": "K decode launches back to back between two HIP events (decode.ms_back_to_back)",
                   "per_call": "K further steps with HIP events around each call (decode.ms_mean/p10/p50/p90, "
                               "quantize_step; event records included)",
                   "instrumented_ms_per_step": instr_ms_step},
        "quantize_bulk": {"tokens": nq, "ms": qms, "tokens_per_s": nq / (qms / 1e3),
                          "GBps": nq * qbpt / (qms / 1e3) / 1e9, "bytes_per_token": qbpt,
                          "frac_hbm_peak": nq * qbpt / (qms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "kernel": "tq_decode_attention (split + reduce kernels)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "frac_of_copy": achieved / copy["GBps"]},
        **extra,
        "page_context": page_context(w, cfg),
        "wall_s_timed": wall,
        "library": tq.version(),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(built, args.cpu_budget)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
