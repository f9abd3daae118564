"""Python binding of libtq (the MI355X TurboQuant KV-cache library).

Argument marshalling only: every step of quantize, decode and dequant runs in
the library's HIP kernels. torch tensors supply device memory and the current
stream. Importing this module loads ``libtq.so`` from this directory and
raises ``ImportError`` when it is missing (build it with
``python compressed_decode_attention_quantize_amd/csrc/build.py``); there is
no fallback path.

The functions mirror include/tq.h:

* ``config_from_preset(name, head_dim)`` / ``config_init(...)`` -> ``Config``
* ``slot_size(cfg, aligned=True)``, ``page_size(cfg, num_kv_heads, block_size)``
* ``layer_signs(cfg, layer_idx)``
* ``quantize_append(cfg, layer_idx, k, v, slot_mapping, kv_pool)``
* ``decode_workspace_size(cfg, batch, num_q_heads, max_seq_len, ring_cap, split_tokens)``
* ``decode_attention(cfg, layer_idx, q, kv_pool, block_tables, seq_lens, max_seq_len, ...)``
* ``dequant(cfg, layer_idx, kv_pool, slot_ids)``
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY names another build of the same library (the sanitizer build
# of the host code that csrc/build.py --sanitize makes); default: the in-tree one
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libtq.so not found at {LIB_PATH}; build it with "
        "`python compressed_decode_attention_quantize_amd/csrc/build.py`")

# torch ships its own HIP runtime (libamdhip64, same soname as ROCm's). It must
# be the one libtq binds to: load torch first so the dynamic linker resolves
# libtq's libamdhip64.so.7 to the already-loaded copy. Two runtimes in one
# process do not share the device ("no ROCm-capable device is detected").
import torch as _torch_for_hip_runtime  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_loaded() -> list:
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes_loaded()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process: " + ", ".join(_hip_runtimes_loaded()) +
                      "; import torch before any other HIP library")

TQ_OK = 0
TQ_ERR_INVALID_ARG = 1
STATUS_NAMES = {0: "TQ_OK", 1: "TQ_ERR_INVALID_ARG", 2: "TQ_ERR_UNKNOWN_PRESET",
                3: "TQ_ERR_UNSUPPORTED", 4: "TQ_ERR_WORKSPACE", 5: "TQ_ERR_HIP"}
F32, BF16, F16 = 0, 1, 2

EXPORTED = ["tq_config_init", "tq_config_from_preset", "tq_layer_config", "tq_boundary_skip_layers",
            "tq_attn_page_size_1_token", "tq_slot_size", "tq_page_size",
            "tq_layer_signs", "tq_quantize_append", "tq_ring_flush", "tq_ring_append", "tq_decode_workspace_size",
            "tq_prefill_workspace_size", "tq_prefill_attention",
            "tq_decode_attention", "tq_decode_attention_no_alloc", "tq_dequant", "tq_check_slot_mapping",
            "tq_check_block_tables", "tq_last_error", "tq_version"]


class Config(ctypes.Structure):
    """Mirror of tq_config (include/tq.h)."""
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("key_quant_bits", ctypes.c_int32),
        ("value_quant_bits", ctypes.c_int32), ("norm_correction", ctypes.c_int32),
        ("seed", ctypes.c_int64),
        ("key_fp8", ctypes.c_int32), ("mse_bits", ctypes.c_int32),
        ("key_mse_bits", ctypes.c_int32), ("centroid_bits", ctypes.c_int32),
        ("n_centroids", ctypes.c_int32), ("key_packed_size", ctypes.c_int32),
        ("value_packed_size", ctypes.c_int32), ("slot_size", ctypes.c_int32),
        ("slot_size_aligned", ctypes.c_int32), ("wht_block", ctypes.c_int32),
        ("centroids", ctypes.c_float * 16), ("midpoints", ctypes.c_float * 15),
        ("centroid_scale", ctypes.c_float),
    ]

    def __repr__(self):
        return (f"Config(head_dim={self.head_dim}, key_quant_bits={self.key_quant_bits}, "
                f"value_quant_bits={self.value_quant_bits}, norm_correction={bool(self.norm_correction)}, "
                f"seed={self.seed}, slot_size_aligned={self.slot_size_aligned})")


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_P = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_CP = ctypes.POINTER(Config)

_lib.tq_config_init.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _CP]
_lib.tq_config_from_preset.argtypes = [ctypes.c_char_p, ctypes.c_int, _CP]
_lib.tq_layer_config.argtypes = [_CP, ctypes.c_int, ctypes.c_int, ctypes.c_int, _CP]
_lib.tq_boundary_skip_layers.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                         ctypes.c_int]
_lib.tq_boundary_skip_layers.restype = ctypes.c_int
_lib.tq_attn_page_size_1_token.argtypes = [_CP, ctypes.c_int, ctypes.c_int]
_lib.tq_attn_page_size_1_token.restype = _i64
_lib.tq_ring_flush.argtypes = [_CP, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, _P, _i64, ctypes.c_int, _P]
_lib.tq_ring_append.argtypes = [_CP, _P, _P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P]
_lib.tq_prefill_workspace_size.argtypes = [_CP, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.POINTER(_sz)]
_lib.tq_prefill_attention.argtypes = [_CP, ctypes.c_int, _P, ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, _P, _i64, ctypes.c_int, _P, ctypes.c_int, _P,
                                      ctypes.c_int, ctypes.c_float, _P, _P, _sz, _P]
_lib.tq_slot_size.argtypes = [_CP, ctypes.c_int]
_lib.tq_slot_size.restype = _i32
_lib.tq_page_size.argtypes = [_CP, ctypes.c_int, ctypes.c_int]
_lib.tq_page_size.restype = _i64
_lib.tq_layer_signs.argtypes = [_CP, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
_lib.tq_quantize_append.argtypes = [_CP, ctypes.c_int, _P, _P, ctypes.c_int, _i64, ctypes.c_int,
                                    _i64, _i64, _P, _P, _i64, ctypes.c_int, _P]
_lib.tq_decode_workspace_size.argtypes = [_CP, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.POINTER(_sz), ctypes.POINTER(ctypes.c_int)]
_lib.tq_decode_attention.argtypes = [_CP, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, _P, _i64, ctypes.c_int, _P, ctypes.c_int, _P,
                                     ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P, _P, _sz,
                                     ctypes.c_int, _P]
_lib.tq_decode_attention_no_alloc.argtypes = [_CP, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _P, _i64, ctypes.c_int, _P, ctypes.c_int, _P,
                                              ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_float, _P,
                                              ctypes.c_int, _P]
_lib.tq_dequant.argtypes = [_CP, ctypes.c_int, _P, _i64, ctypes.c_int, ctypes.c_int, _P, _i64, _P, _P, _P]
_lib.tq_check_slot_mapping.argtypes = [_P, _i64, _i64, ctypes.c_int, ctypes.POINTER(_i64)]
_lib.tq_check_block_tables.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _i64, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
for _name in ("tq_config_init", "tq_config_from_preset", "tq_layer_config", "tq_layer_signs", "tq_quantize_append",
              "tq_ring_flush", "tq_ring_append", "tq_prefill_workspace_size", "tq_prefill_attention",
              "tq_decode_workspace_size", "tq_decode_attention", "tq_decode_attention_no_alloc", "tq_dequant",
              "tq_check_slot_mapping", "tq_check_block_tables"):
    getattr(_lib, _name).restype = ctypes.c_int
_lib.tq_last_error.restype = ctypes.c_char_p
_lib.tq_version.restype = ctypes.c_char_p


def lib() -> ctypes.CDLL:
    return _lib


def last_error() -> str:
    return _lib.tq_last_error().decode()


def version() -> str:
    return _lib.tq_version().decode()


def _check(status: int) -> None:
    if status != TQ_OK:
        raise TQError(status, last_error())


# ----------------------------------------------------------------------------- config

def config_init(head_dim: int, key_bits: int, value_bits: int, norm_correction: bool = False,
                seed: int = 42) -> Config:
    c = Config()
    _check(_lib.tq_config_init(head_dim, key_bits, value_bits, int(bool(norm_correction)), seed,
                               ctypes.byref(c)))
    return c


def config_from_preset(preset: str, head_dim: int) -> Config:
    c = Config()
    _check(_lib.tq_config_from_preset(preset.encode(), head_dim, ctypes.byref(c)))
    return c


def layer_config(base: Config, layer_idx: int, initial_layers: int = 4,
                 initial_layers_key_bits: int = 0) -> Config:
    """Config of one layer under layer-adaptive key bits (0 = base bits + 1)."""
    c = Config()
    _check(_lib.tq_layer_config(ctypes.byref(base), layer_idx, initial_layers, initial_layers_key_bits,
                                ctypes.byref(c)))
    return c


def boundary_skip_layers(num_layers: int, n: int = 2, hybrid: bool = False) -> list:
    """Layer indices (as strings) that keep the unquantized cache."""
    cnt = _lib.tq_boundary_skip_layers(num_layers, n, int(bool(hybrid)), None, 0)
    if cnt < 0:
        raise TQError(1, last_error())
    buf = (ctypes.c_int32 * max(cnt, 1))()
    _lib.tq_boundary_skip_layers(num_layers, n, int(bool(hybrid)), buf, cnt)
    return [str(buf[i]) for i in range(cnt)]


def attn_page_size_1_token(cfg: Config, num_kv_heads: int, skip_dtype_bytes: int = 0) -> int:
    n = _lib.tq_attn_page_size_1_token(ctypes.byref(cfg), num_kv_heads, skip_dtype_bytes)
    if n < 0:
        raise TQError(1, last_error())
    return n


def slot_size(cfg: Config, aligned: bool = True) -> int:
    n = _lib.tq_slot_size(ctypes.byref(cfg), int(aligned))
    if n < 0:
        raise TQError(1, last_error())
    return n


def page_size(cfg: Config, num_kv_heads: int, block_size: int) -> int:
    n = _lib.tq_page_size(ctypes.byref(cfg), num_kv_heads, block_size)
    if n < 0:
        raise TQError(1, last_error())
    return n


def layer_signs(cfg: Config, layer_idx: int):
    import numpy as np
    out = (ctypes.c_float * cfg.head_dim)()
    _check(_lib.tq_layer_signs(ctypes.byref(cfg), layer_idx, out))
    return np.frombuffer(out, dtype=np.float32).copy()


# ----------------------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16, float16)")


def _dev(t, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream_ptr(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _alloc_stream(stream, device):
    """Context for allocating a call's own out / workspace tensors: on the
    stream the call runs on. torch's caching allocator hands a freed block
    only to later allocations on the stream it was allocated on, so memory
    the kernels of a caller-chosen stream still use is never given to work
    on another stream."""
    import contextlib
    torch = _torch()
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device))


def quantize_append(cfg: Config, layer_idx: int, k, v, slot_mapping, kv_pool, stream=None) -> None:
    """k, v: [T, Hkv, D] (or [T, Hkv*D] rows with a token stride) float32/bf16/f16
    with the head and element dims contiguous; slot_mapping int64 [T];
    kv_pool uint8 [num_blocks, Hkv, block_size, S]."""
    torch = _torch()
    _dev(k, "k")
    _dev(v, "v")
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(kv_pool, "kv_pool", torch.uint8)
    if k.dtype != v.dtype:
        raise TypeError("k and v must have the same dtype")
    if kv_pool.dim() != 4 or kv_pool.shape[3] != cfg.slot_size_aligned or not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous [num_blocks, Hkv, block_size, slot_size_aligned]")
    t_count = k.shape[0]
    hkv = kv_pool.shape[1]
    for name, x in (("k", k), ("v", v)):
        if x.dim() != 3 or x.shape[1] != hkv or x.shape[2] != cfg.head_dim:
            raise ValueError(f"{name} must be [T, {hkv}, {cfg.head_dim}]")
        if x.stride(2) != 1 or x.stride(1) != cfg.head_dim:
            raise ValueError(f"{name}: heads and elements must be contiguous")
    if v.shape[0] != t_count or slot_mapping.shape != (t_count,) or not slot_mapping.is_contiguous():
        raise ValueError("k, v and slot_mapping disagree on the token count")
    s = stream if stream is not None else _stream_ptr(k)
    _check(_lib.tq_quantize_append(ctypes.byref(cfg), layer_idx, k.data_ptr(), v.data_ptr(), _dtype_code(k),
                                   t_count, hkv, k.stride(0) if t_count > 1 else hkv * cfg.head_dim,
                                   v.stride(0) if t_count > 1 else hkv * cfg.head_dim,
                                   slot_mapping.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0],
                                   kv_pool.shape[2], s))


def ring_flush(cfg: Config, layer_idx: int, ring_k, ring_v, ring_lens, seq_lens, block_tables, kv_pool,
               stream=None) -> None:
    """Compress every full ring (bf16 [B, Hkv, cap, D]) into the pool at its
    sequence's next positions; updates ring_lens / seq_lens (int32 [B]) in place."""
    torch = _torch()
    _dev(ring_k, "ring_k", torch.bfloat16)
    _dev(ring_v, "ring_v", torch.bfloat16)
    _dev(ring_lens, "ring_lens", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(kv_pool, "kv_pool", torch.uint8)
    if ring_k.dim() != 4 or ring_k.shape != ring_v.shape or ring_k.shape[3] != cfg.head_dim \
            or not ring_k.is_contiguous() or not ring_v.is_contiguous():
        raise ValueError(f"ring_k/ring_v must be contiguous bf16 [B, Hkv, cap, {cfg.head_dim}]")
    bsz, hkv, cap, _ = ring_k.shape
    if ring_lens.shape != (bsz,) or seq_lens.shape != (bsz,) or block_tables.dim() != 2 \
            or block_tables.shape[0] != bsz or not block_tables.is_contiguous():
        raise ValueError("ring_lens/seq_lens must be [B] and block_tables contiguous [B, max_blocks]")
    if kv_pool.dim() != 4 or kv_pool.shape[1] != hkv or kv_pool.shape[3] != cfg.slot_size_aligned \
            or not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous [num_blocks, Hkv, block_size, slot_size_aligned]")
    s = stream if stream is not None else _stream_ptr(ring_k)
    _check(_lib.tq_ring_flush(ctypes.byref(cfg), layer_idx, ring_k.data_ptr(), ring_v.data_ptr(), cap,
                              ring_lens.data_ptr(), seq_lens.data_ptr(), block_tables.data_ptr(),
                              block_tables.shape[1], bsz, hkv, kv_pool.data_ptr(), kv_pool.shape[0],
                              kv_pool.shape[2], s))


def ring_append(cfg: Config, k_new, v_new, ring_k, ring_v, ring_lens, stream=None) -> None:
    """Copy each sequence's new token (bf16 [B, Hkv, D]) to the end of its ring."""
    torch = _torch()
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (ring_k, "ring_k"), (ring_v, "ring_v")):
        _dev(t, n, torch.bfloat16)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    _dev(ring_lens, "ring_lens", torch.int32)
    bsz, hkv, cap, d = ring_k.shape
    if k_new.shape != (bsz, hkv, d) or v_new.shape != k_new.shape or ring_v.shape != ring_k.shape \
            or d != cfg.head_dim or ring_lens.shape != (bsz,):
        raise ValueError("k_new/v_new must be [B, Hkv, D] matching the ring [B, Hkv, cap, D]")
    s = stream if stream is not None else _stream_ptr(ring_k)
    _check(_lib.tq_ring_append(ctypes.byref(cfg), k_new.data_ptr(), v_new.data_ptr(), bsz, hkv, ring_k.data_ptr(),
                               ring_v.data_ptr(), cap, ring_lens.data_ptr(), s))


def ring_step(cfg: Config, layer_idx: int, k_new, v_new, ring_k, ring_v, ring_lens, seq_lens, block_tables,
              kv_pool, stream=None) -> None:
    """One decode step's write: flush full rings as whole chunks, then append."""
    ring_flush(cfg, layer_idx, ring_k, ring_v, ring_lens, seq_lens, block_tables, kv_pool, stream)
    ring_append(cfg, k_new, v_new, ring_k, ring_v, ring_lens, stream)


def decode_workspace_size(cfg: Config, batch: int, num_q_heads: int, max_seq_len: int,
                          ring_cap: int = 0, split_tokens: int = 0):
    """Returns (bytes, chunks per sequence)."""
    b = _sz()
    n = ctypes.c_int()
    _check(_lib.tq_decode_workspace_size(ctypes.byref(cfg), batch, num_q_heads, max_seq_len, ring_cap,
                                         split_tokens, ctypes.byref(b), ctypes.byref(n)))
    return b.value, n.value


def _decode_args(cfg: Config, q, kv_pool, block_tables, seq_lens, ring_k, ring_v, ring_lens):
    """Checks the tensors of a decode call; returns (batch, Hq, Hkv, D,
    ring_cap, ring pointers)."""
    torch = _torch()
    _dev(q, "q")
    _dev(kv_pool, "kv_pool", torch.uint8)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if not q.is_contiguous() or q.dim() != 3 or q.shape[2] != cfg.head_dim:
        raise ValueError(f"q must be contiguous [B, Hq, {cfg.head_dim}]")
    if kv_pool.dim() != 4 or kv_pool.shape[3] != cfg.slot_size_aligned or not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous [num_blocks, Hkv, block_size, slot_size_aligned]")
    bsz, hq, d = q.shape
    hkv = kv_pool.shape[1]
    if block_tables.dim() != 2 or block_tables.shape[0] != bsz or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous [B, max_blocks]")
    if seq_lens.shape != (bsz,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be [B]")
    ring_cap = 0
    rk = rv = rl = None
    if ring_k is not None:
        _dev(ring_k, "ring_k", torch.bfloat16)
        _dev(ring_v, "ring_v", torch.bfloat16)
        _dev(ring_lens, "ring_lens", torch.int32)
        if ring_k.shape != ring_v.shape or ring_k.dim() != 4 or ring_k.shape[:2] != (bsz, hkv) \
                or ring_k.shape[3] != d or not ring_k.is_contiguous() or not ring_v.is_contiguous():
            raise ValueError(f"ring_k/ring_v must be contiguous bf16 [B, {hkv}, ring_cap, {d}]")
        ring_cap = ring_k.shape[2]
        rk, rv, rl = ring_k.data_ptr(), ring_v.data_ptr(), ring_lens.data_ptr()
    return bsz, hq, hkv, d, ring_cap, rk, rv, rl


def decode_attention(cfg: Config, layer_idx: int, q, kv_pool, block_tables, seq_lens, max_seq_len: int,
                     ring_k=None, ring_v=None, ring_lens=None, softmax_scale: float = 0.0,
                     out=None, workspace=None, split_tokens: int = 0, stream=None):
    """q [B, Hq, D] (f32/bf16/f16, contiguous) -> out [B, Hq, D] float32.

    block_tables int32 [B, max_blocks]; seq_lens int32 [B]; ring_k/ring_v
    bf16 [B, Hkv, ring_cap, D] with ring_lens int32 [B], or None.
    """
    torch = _torch()
    bsz, hq, hkv, d, ring_cap, rk, rv, rl = _decode_args(cfg, q, kv_pool, block_tables, seq_lens,
                                                         ring_k, ring_v, ring_lens)
    need, _ = decode_workspace_size(cfg, bsz, hq, max_seq_len, ring_cap, split_tokens)
    with _alloc_stream(stream, q.device):
        if out is None:
            out = torch.empty((bsz, hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(out, "out", torch.float32)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 like q")
    _dev(workspace, "workspace", torch.uint8)
    s = stream if stream is not None else _stream_ptr(q)
    _check(_lib.tq_decode_attention(ctypes.byref(cfg), layer_idx, q.data_ptr(), _dtype_code(q), bsz, hq, hkv,
                                    kv_pool.data_ptr(), kv_pool.shape[0], kv_pool.shape[2],
                                    block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(),
                                    max_seq_len, rk, rv, rl, ring_cap, float(softmax_scale), out.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(), split_tokens, s))
    return out


def decode_attention_no_alloc(cfg: Config, layer_idx: int, q, kv_pool, block_tables, seq_lens, max_seq_len: int,
                              out, ring_k=None, ring_v=None, ring_lens=None, softmax_scale: float = 0.0,
                              split_tokens: int = 0, stream=None):
    """decode_attention through tq_decode_attention_no_alloc: the caller
    passes `out` (float32 [B, Hq, D]); the library's per-device static
    scratch takes the workspace's place, so nothing is allocated. Calls that
    overlap on one device race."""
    torch = _torch()
    bsz, hq, hkv, d, ring_cap, rk, rv, rl = _decode_args(cfg, q, kv_pool, block_tables, seq_lens,
                                                         ring_k, ring_v, ring_lens)
    _dev(out, "out", torch.float32)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 like q")
    s = stream if stream is not None else _stream_ptr(q)
    _check(_lib.tq_decode_attention_no_alloc(ctypes.byref(cfg), layer_idx, q.data_ptr(), _dtype_code(q), bsz, hq,
                                             hkv, kv_pool.data_ptr(), kv_pool.shape[0], kv_pool.shape[2],
                                             block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(),
                                             max_seq_len, rk, rv, rl, ring_cap, float(softmax_scale),
                                             out.data_ptr(), split_tokens, s))
    return out


def prefill_workspace_size(cfg: Config, batch: int, num_q_heads: int, num_kv_heads: int, max_chunk: int,
                           max_hist: int, max_blocks_per_seq: int, q_dtype: int = BF16) -> int:
    n = _sz(0)
    _check(_lib.tq_prefill_workspace_size(ctypes.byref(cfg), batch, num_q_heads, num_kv_heads, max_chunk, max_hist,
                                          max_blocks_per_seq, q_dtype, ctypes.byref(n)))
    return n.value


def prefill_attention(cfg: Config, layer_idx: int, q, k_chunk, v_chunk, cu_chunk, max_chunk: int, kv_pool,
                      block_tables, hist_lens, max_hist: int, softmax_scale: float = 0.0, out=None, workspace=None,
                      stream=None):
    """Continuation prefill: q [N, Hq, D] (f32/bf16/f16), k_chunk / v_chunk bf16
    [N, Hkv, D], cu_chunk int32 [B + 1], hist_lens int32 [B] -> out [N, Hq, D] fp32."""
    torch = _torch()
    _dev(q, "q")
    _dev(k_chunk, "k_chunk", torch.bfloat16)
    _dev(v_chunk, "v_chunk", torch.bfloat16)
    _dev(cu_chunk, "cu_chunk", torch.int32)
    _dev(hist_lens, "hist_lens", torch.int32)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(kv_pool, "kv_pool", torch.uint8)
    if q.dim() != 3 or q.shape[2] != cfg.head_dim or not q.is_contiguous():
        raise ValueError(f"q must be contiguous [N, Hq, {cfg.head_dim}]")
    n, hq, d = q.shape
    hkv = kv_pool.shape[1]
    if k_chunk.shape != (n, hkv, d) or v_chunk.shape != k_chunk.shape or not k_chunk.is_contiguous() \
            or not v_chunk.is_contiguous():
        raise ValueError(f"k_chunk/v_chunk must be contiguous bf16 [N, {hkv}, {d}]")
    bsz = hist_lens.shape[0]
    if cu_chunk.shape != (bsz + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != bsz \
            or not block_tables.is_contiguous():
        raise ValueError("cu_chunk must be [B + 1], hist_lens [B], block_tables contiguous [B, max_blocks]")
    if kv_pool.dim() != 4 or kv_pool.shape[3] != cfg.slot_size_aligned or not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous [num_blocks, Hkv, block_size, slot_size_aligned]")
    need = prefill_workspace_size(cfg, bsz, hq, hkv, max_chunk, max_hist, block_tables.shape[1], _dtype_code(q))
    with _alloc_stream(stream, q.device):
        if out is None:
            out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(out, "out", torch.float32)
    _dev(workspace, "workspace", torch.uint8)
    s = stream if stream is not None else _stream_ptr(q)
    _check(_lib.tq_prefill_attention(ctypes.byref(cfg), layer_idx, q.data_ptr(), _dtype_code(q), k_chunk.data_ptr(),
                                     v_chunk.data_ptr(), cu_chunk.data_ptr(), bsz, max_chunk, hq, hkv,
                                     kv_pool.data_ptr(), kv_pool.shape[0], kv_pool.shape[2], block_tables.data_ptr(),
                                     block_tables.shape[1], hist_lens.data_ptr(), max_hist, float(softmax_scale),
                                     out.data_ptr(), workspace.data_ptr(), workspace.numel(), s))
    return out


def dequant(cfg: Config, layer_idx: int, kv_pool, slot_ids, k_out=None, v_out=None, stream=None):
    """slot_ids int64 [n] -> (K_hat, V_hat) float32 [n, Hkv, D] in the original basis."""
    torch = _torch()
    _dev(kv_pool, "kv_pool", torch.uint8)
    _dev(slot_ids, "slot_ids", torch.int64)
    if kv_pool.dim() != 4 or kv_pool.shape[3] != cfg.slot_size_aligned or not kv_pool.is_contiguous():
        raise ValueError("kv_pool must be contiguous [num_blocks, Hkv, block_size, slot_size_aligned]")
    n = slot_ids.numel()
    hkv = kv_pool.shape[1]
    shape = (n, hkv, cfg.head_dim)
    with _alloc_stream(stream, kv_pool.device):
        if k_out is None:
            k_out = torch.empty(shape, dtype=torch.float32, device=kv_pool.device)
        if v_out is None:
            v_out = torch.empty(shape, dtype=torch.float32, device=kv_pool.device)
    s = stream if stream is not None else _stream_ptr(kv_pool)
    _check(_lib.tq_dequant(ctypes.byref(cfg), layer_idx, kv_pool.data_ptr(), kv_pool.shape[0], hkv,
                           kv_pool.shape[2], slot_ids.data_ptr(), n, k_out.data_ptr(), v_out.data_ptr(), s))
    return k_out, v_out


# ----------------------------------------------------------------------------- prepared calls

def _host_array(a, dtype):
    """A contiguous host (numpy) copy of a numpy array or torch tensor."""
    import numpy as np
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def check_slot_mapping(slot_mapping, num_blocks: int, block_size: int) -> None:
    """Debug check (host copy): every entry is -1 or a slot of the pool, and no
    slot is written twice. Raises TQError naming the first offending token
    (its index also in the exception's `index`)."""
    import numpy as np
    m = _host_array(slot_mapping, np.int64).reshape(-1)
    bad = _i64(-1)
    st = _lib.tq_check_slot_mapping(m.ctypes.data if m.size else None, m.size, num_blocks, block_size,
                                    ctypes.byref(bad))
    if st != TQ_OK:
        e = TQError(st, last_error())
        e.index = bad.value
        raise e


def check_block_tables(block_tables, seq_lens, num_blocks: int, block_size: int) -> None:
    """Debug check (host copies): each sequence's blocks fit its table row and
    their ids lie in the pool. Raises TQError naming the first offending
    (sequence, logical block), also in the exception's `seq` and `block`."""
    import numpy as np
    t = _host_array(block_tables, np.int32)
    n = _host_array(seq_lens, np.int32).reshape(-1)
    if t.ndim != 2 or t.shape[0] != n.size:
        raise ValueError("block_tables [batch, max_blocks] and seq_lens [batch] required")
    bs_, bb = ctypes.c_int(-1), ctypes.c_int(-1)
    st = _lib.tq_check_block_tables(t.ctypes.data if t.size else None, n.size, t.shape[1],
                                    n.ctypes.data if n.size else None, num_blocks, block_size,
                                    ctypes.byref(bs_), ctypes.byref(bb))
    if st != TQ_OK:
        e = TQError(st, last_error())
        e.seq, e.block = bs_.value, bb.value
        raise e


class _Prepared:
    """A library call with its arguments marshalled once; calling it issues
    the same C call again (for tight loops where per-call validation in
    Python would dominate). The tensors must stay alive and unchanged in
    shape while the object is used."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != TQ_OK:
            raise TQError(st, last_error())


def prepare_quantize(cfg: Config, layer_idx: int, k, v, slot_mapping, kv_pool, stream=None) -> _Prepared:
    """Validated once like quantize_append; returns a callable re-issuing it."""
    quantize_append(cfg, layer_idx, k[:0], v[:0], slot_mapping[:0], kv_pool, stream)  # validates shapes/dtypes
    torch = _torch()
    _dev(k, "k"); _dev(v, "v"); _dev(slot_mapping, "slot_mapping", torch.int64)
    t_count = k.shape[0]
    hkv = kv_pool.shape[1]
    if k.dim() != 3 or k.shape[1:] != (hkv, cfg.head_dim) or v.shape != k.shape or slot_mapping.shape != (t_count,):
        raise ValueError("k, v [T, Hkv, D] and slot_mapping [T] required")
    s = stream if stream is not None else _stream_ptr(k)
    args = (ctypes.byref(cfg), layer_idx, k.data_ptr(), v.data_ptr(), _dtype_code(k), t_count, hkv,
            k.stride(0) if t_count > 1 else hkv * cfg.head_dim, v.stride(0) if t_count > 1 else hkv * cfg.head_dim,
            slot_mapping.data_ptr(), kv_pool.data_ptr(), kv_pool.shape[0], kv_pool.shape[2], s)
    return _Prepared(_lib.tq_quantize_append, args, (cfg, k, v, slot_mapping, kv_pool))


def prepare_decode(cfg: Config, layer_idx: int, q, kv_pool, block_tables, seq_lens, max_seq_len: int,
                   ring_k=None, ring_v=None, ring_lens=None, softmax_scale: float = 0.0, out=None,
                   workspace=None, split_tokens: int = 0, stream=None) -> _Prepared:
    """Validated once like decode_attention (which it runs once); returns a
    callable re-issuing the same call into the same out/workspace."""
    torch = _torch()
    bsz, hq, d = q.shape
    ring_cap = 0 if ring_k is None else ring_k.shape[2]
    need, _ = decode_workspace_size(cfg, bsz, hq, max_seq_len, ring_cap, split_tokens)
    with _alloc_stream(stream, q.device):
        if out is None:
            out = torch.empty((bsz, hq, d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    decode_attention(cfg, layer_idx, q, kv_pool, block_tables, seq_lens, max_seq_len, ring_k, ring_v,
                     ring_lens, softmax_scale, out, workspace, split_tokens, stream)
    s = stream if stream is not None else _stream_ptr(q)
    rk = None if ring_k is None else ring_k.data_ptr()
    rv = None if ring_v is None else ring_v.data_ptr()
    rl = None if ring_lens is None else ring_lens.data_ptr()
    args = (ctypes.byref(cfg), layer_idx, q.data_ptr(), _dtype_code(q), bsz, hq, kv_pool.shape[1],
            kv_pool.data_ptr(), kv_pool.shape[0], kv_pool.shape[2], block_tables.data_ptr(),
            block_tables.shape[1], seq_lens.data_ptr(), max_seq_len, rk, rv, rl, ring_cap,
            ctypes.c_float(softmax_scale), out.data_ptr(), workspace.data_ptr(), workspace.numel(),
            split_tokens, s)
    p = _Prepared(_lib.tq_decode_attention, args,
                  (cfg, q, kv_pool, block_tables, seq_lens, ring_k, ring_v, ring_lens, out, workspace))
    p.out = out
    p.workspace = workspace
    return p
