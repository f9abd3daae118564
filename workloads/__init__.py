"""Seeded synthetic inputs for the TurboQuant decode path.

Shared by the tests and bench.py; holds no arithmetic of the method (no
rotation, quantization or attention), only random data, lengths and paged
block tables. Neither the oracle nor the library imports it.

Workloads (the five configurations the library is measured and tested on):

* ``tiny``    D=64, 2 KV / 4 q heads, one sequence of 512 tokens (511 bulk
              appended, then 1), 3-bit keys + 4-bit values, seed 42; K, V, q
              fp32 N(0,1) from numpy.default_rng(42); identity block table.
* ``k8v4``    turboquant_k8v4, D=128, 32 q / 8 KV heads, 16 sequences x 8192.
* ``4bit_nc`` turboquant_4bit_nc, D=128, 32/8, 64 x 32768.
* ``3bit_nc`` turboquant_3bit_nc, D=128, 64/8, 8 sequences x (130944
              compressed + a full 128-token bf16 ring) = 131072.
* ``k3v4_nc`` turboquant_k3v4_nc, D=96, 16/4, 64 sequences with log-normal
              lengths (median 4096, sigma 1, clipped to [16, 65536], the first
              one set to 65536), plus a concurrent 65536-token prefill.
* ``k3v2_nc`` 3-bit MSE keys + 2-bit values with norm correction (the
              bit-width variant), D=128, 32/8, 64 x 32768 (the 4bit_nc shape).
* ``prefill_4bit_nc`` continuation prefill: turboquant_4bit_nc, D=128, 32/8,
              4 sequences with 32768 compressed tokens each and a new
              512-token chunk each (bf16 q, K, V of the same recipe).

K/V recipe for the D=128 workloads: bf16 N(0,1) with 4 outlier channels per
KV head scaled x10 (channel sets drawn per head, independently for K and V);
for k3v4_nc: bf16 Student-t with 4 degrees of freedom. q: bf16 N(0,1).
Block tables: a random permutation of the pool's blocks, handed out to the
sequences in logical order.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    preset: str | None          # None: explicit bits below
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    batch: int
    context: int                # attended tokens per sequence (max for log-normal)
    ring: int = 0               # ring tokens per sequence (included in context)
    key_bits: int = 3
    value_bits: int = 4
    norm_correction: bool = False
    dist: str = "normal_outliers"   # "normal", "normal_outliers", "student_t"
    lognormal_lengths: bool = False
    prefill_tokens: int = 0     # concurrent prefill append (k3v4_nc)
    seed: int = 0
    block_size: int = 16
    in_dtype: str = "bf16"
    chunk: int = 0              # continuation-prefill chunk tokens per sequence (prefill workloads)
    description: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", None, 64, 4, 2, 1, 512, key_bits=3, value_bits=4, dist="normal",
                     seed=42, in_dtype="f32",
                     description="1 seq, D=64, 4q/2kv, ctx 512, k3/v4, fp32 N(0,1)"),
    "k8v4": Workload("k8v4", "turboquant_k8v4", 128, 32, 8, 16, 8192, seed=1002,
                     description="turboquant_k8v4, D=128, 32q/8kv, batch 16, ctx 8192"),
    "4bit_nc": Workload("4bit_nc", "turboquant_4bit_nc", 128, 32, 8, 64, 32768, seed=1003,
                        description="turboquant_4bit_nc, D=128, 32q/8kv, batch 64, ctx 32768"),
    "3bit_nc": Workload("3bit_nc", "turboquant_3bit_nc", 128, 64, 8, 8, 131072, ring=128, seed=1004,
                        description="turboquant_3bit_nc, D=128, 64q/8kv, batch 8, ctx 131072 (128 in ring)"),
    "k3v4_nc": Workload("k3v4_nc", "turboquant_k3v4_nc", 96, 16, 4, 64, 65536, dist="student_t",
                        lognormal_lengths=True, prefill_tokens=65536, seed=1005,
                        description="turboquant_k3v4_nc, D=96, 16q/4kv, 64 log-normal seqs (median 4096, max 65536) + 65536-token prefill"),
    "prefill_4bit_nc": Workload("prefill_4bit_nc", "turboquant_4bit_nc", 128, 32, 8, 4, 32768, seed=1007, chunk=512,
                                description="continuation prefill, turboquant_4bit_nc, D=128, 32q/8kv, 4 seqs x "
                                            "32768 compressed history + 512-token chunk each"),
    "k3v2_nc": Workload("k3v2_nc", None, 128, 32, 8, 64, 32768, key_bits=3, value_bits=2,
                        norm_correction=True, seed=1006,
                        description="3-bit MSE keys + 2-bit values + NC, D=128, 32q/8kv, batch 64, ctx 32768"),
}


def scaled(w: Workload, batch: int | None = None, context: int | None = None, **kw) -> Workload:
    """Same recipe at smaller sizes (for parity tests)."""
    from dataclasses import replace
    args = {}
    if batch is not None:
        args["batch"] = batch
    if context is not None:
        args["context"] = context
    args.update(kw)
    return replace(w, **args)


def sequence_lengths(w: Workload) -> np.ndarray:
    """Compressed tokens per sequence (context minus the ring)."""
    if not w.lognormal_lengths:
        return np.full(w.batch, w.context - w.ring, dtype=np.int64)
    rng = np.random.default_rng(w.seed)
    raw = np.exp(rng.normal(math.log(4096.0), 1.0, size=w.batch))
    lens = np.clip(np.rint(raw), 16, w.context).astype(np.int64)
    lens[0] = w.context
    return lens - w.ring


def block_tables(w: Workload, lens: np.ndarray, extra_blocks: int = 0):
    """(tables int32 [B, max_blocks], num_blocks): a random permutation of all
    blocks handed out to the sequences in logical order."""
    bs = w.block_size
    nblk = [max(1, math.ceil(int(n) / bs)) for n in lens]
    total = sum(nblk) + extra_blocks
    rng = np.random.default_rng(w.seed + 7)
    perm = rng.permutation(total).astype(np.int32)
    tables = np.zeros((len(lens), max(nblk)), dtype=np.int32)
    used = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[used:used + n]
        used += n
    return tables, total, perm[used:]


def slot_ids_for(tables: np.ndarray, b: int, start: int, count: int, block_size: int) -> np.ndarray:
    pos = np.arange(start, start + count, dtype=np.int64)
    return tables[b, pos // block_size].astype(np.int64) * block_size + pos % block_size


# ---------------------------------------------------------------------------- torch data

def _torch():
    import torch
    return torch


def torch_dtype(name: str):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


class KVSource:
    """Deterministic K/V/q generator for one workload on one device.

    Outlier channels are fixed per KV head; token rows are drawn in the order
    they are requested, so the same sequence of requests gives the same data.
    """

    def __init__(self, w: Workload, device, stream_id: int = 0):
        torch = _torch()
        self.w = w
        self.device = torch.device(device)
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(w.seed * 1000 + stream_id)
        d, h = w.head_dim, w.num_kv_heads
        self.k_scale = torch.ones((h, d), device=self.device)
        self.v_scale = torch.ones((h, d), device=self.device)
        if w.dist == "normal_outliers":
            for head in range(h):
                kc = torch.randperm(d, generator=self.gen, device=self.device)[:4]
                vc = torch.randperm(d, generator=self.gen, device=self.device)[:4]
                self.k_scale[head, kc] = 10.0
                self.v_scale[head, vc] = 10.0

    def _draw(self, shape):
        torch = _torch()
        if self.w.dist == "student_t":
            z = torch.randn(shape, generator=self.gen, device=self.device)
            # chi-square with 4 degrees of freedom as a sum of 4 squared normals
            c = torch.randn((4, *shape), generator=self.gen, device=self.device).pow(2).sum(0)
            return z / torch.sqrt(c / 4.0)
        return torch.randn(shape, generator=self.gen, device=self.device)

    def kv(self, n_tokens: int):
        """K, V [n_tokens, Hkv, D] in the workload's input dtype."""
        w = self.w
        shape = (n_tokens, w.num_kv_heads, w.head_dim)
        k = self._draw(shape) * self.k_scale
        v = self._draw(shape) * self.v_scale
        dt = torch_dtype(w.in_dtype)
        return k.to(dt), v.to(dt)

    def q(self, batch: int | None = None):
        w = self.w
        b = w.batch if batch is None else batch
        return self._draw((b, w.num_q_heads, w.head_dim)).to(torch_dtype(w.in_dtype))

    def ring(self, batch: int | None = None):
        w = self.w
        b = w.batch if batch is None else batch
        torch = _torch()
        shape = (b, w.num_kv_heads, max(w.ring, 1), w.head_dim)
        k = (self._draw(shape) * self.k_scale[None, :, None, :]).to(torch.bfloat16)
        v = (self._draw(shape) * self.v_scale[None, :, None, :]).to(torch.bfloat16)
        return k, v


def tiny_numpy():
    """The tiny workload's data exactly: (K [512,2,64], V [512,2,64], q [1,4,64]) fp32."""
    rng = np.random.default_rng(42)
    k = rng.standard_normal((512, 2, 64)).astype(np.float32)
    v = rng.standard_normal((512, 2, 64)).astype(np.float32)
    q = rng.standard_normal((1, 4, 64)).astype(np.float32)
    return k, v, q
