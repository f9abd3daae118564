"""CPU tests of the C-ABI library: it loads without a GPU, exports every symbol
include/tq.h declares, its host-side config arithmetic and tables equal the
oracle's bit for bit, and argument errors are reported before anything is
launched. No GPU work is enqueued here."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import config as OC
from oracle import lloyd_max as OL
from oracle import rotation as OR
from tests.conftest import ROOT

tq = pytest.importorskip("compressed_decode_attention_quantize_amd",
                         reason="libtq.so not built (run __graft_entry__.build())")


def test_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "tq.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(tq_[a-z_0-9]+)\s*\(", header, re.M))
    assert {"tq_config_init", "tq_quantize_append", "tq_decode_attention", "tq_dequant"} <= declared
    for name in declared:
        assert hasattr(tq.lib(), name), name
    assert set(tq.EXPORTED) == declared


PRESETS = ["turboquant_k8v4", "turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"]


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("d", [64, 96, 128])
def test_preset_config_matches_oracle(preset, d):
    c = tq.config_from_preset(preset, d)
    o = OC.from_cache_dtype(preset, d)
    for f in ("head_dim", "key_quant_bits", "value_quant_bits", "seed", "key_packed_size",
              "value_packed_size", "slot_size", "slot_size_aligned", "mse_bits", "key_mse_bits",
              "centroid_bits", "n_centroids", "wht_block"):
        assert getattr(c, f) == int(getattr(o, f)), f
    assert bool(c.norm_correction) == o.norm_correction and bool(c.key_fp8) == o.key_fp8
    assert tq.slot_size(c) == o.slot_size_aligned and tq.slot_size(c, aligned=False) == o.slot_size
    assert tq.page_size(c, 8, 16) == 16 * 8 * o.slot_size_aligned


@pytest.mark.parametrize("kb,vb", [(3, 2), (4, 2), (8, 2), (3, 3), (8, 3)])
@pytest.mark.parametrize("d", [64, 96, 128])
def test_custom_bits_config_matches_oracle(d, kb, vb):
    c = tq.config_init(d, kb, vb, True, 42)
    o = OC.TQConfig(head_dim=d, key_quant_bits=kb, value_quant_bits=vb, norm_correction=True)
    for f in ("key_packed_size", "value_packed_size", "slot_size", "slot_size_aligned", "mse_bits",
              "key_mse_bits", "n_centroids", "wht_block"):
        assert getattr(c, f) == int(getattr(o, f)), f
    c32, m32 = OL.tables_f32(d, o.mse_bits)
    assert np.array_equal(np.array(list(c.centroids), np.float32)[: o.n_centroids].view(np.uint32),
                          c32.view(np.uint32))
    assert np.array_equal(np.array(list(c.midpoints), np.float32)[: o.n_centroids - 1].view(np.uint32),
                          m32.view(np.uint32))


@pytest.mark.parametrize("preset", PRESETS + ["k3v2"])
@pytest.mark.parametrize("layer", [0, 3, 4, 9])
@pytest.mark.parametrize("initial_bits", [0, 4, 8])
def test_layer_config_matches_oracle(preset, layer, initial_bits):
    if preset == "k3v2":
        base = tq.config_init(128, 3, 2, True, 42)
        obase = OC.TQConfig(head_dim=128, key_quant_bits=3, value_quant_bits=2, norm_correction=True)
    else:
        base = tq.config_from_preset(preset, 128)
        obase = OC.from_cache_dtype(preset, 128)
    want = OC.layer_config(obase, layer, initial_layers_key_bits=initial_bits or None)
    if want.key_quant_bits not in (3, 4, 8):   # e.g. 5 bits from a 4-bit base: not built
        with pytest.raises(tq.TQError) as ei:
            tq.layer_config(base, layer, 4, initial_bits)
        assert ei.value.status == 1
        return
    c = tq.layer_config(base, layer, 4, initial_bits)
    for f in ("head_dim", "key_quant_bits", "value_quant_bits", "seed", "slot_size_aligned", "n_centroids"):
        assert getattr(c, f) == int(getattr(want, f)), f
    assert bool(c.norm_correction) == want.norm_correction
    assert np.array_equal(np.array(list(c.centroids), np.float32)[: want.n_centroids],
                          OL.tables_f32(128, want.mse_bits)[0])


def test_layer_config_argument_errors():
    base = tq.config_from_preset("turboquant_k3v4_nc", 128)
    for args in ((-1, 4, 0), (0, -1, 0), (0, 4, -2)):
        with pytest.raises(tq.TQError) as ei:
            tq.layer_config(base, *args)
        assert ei.value.status == 1
    assert tq.layer_config(base, 0, 0, 0).key_quant_bits == 3   # no initial layers


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("bits", [3, 4])
def test_tables_bit_equal_to_oracle(d, bits):
    c = tq.config_init(d, bits, 4, False, 42)
    c32, m32 = OL.tables_f32(d, bits)
    got_c = np.array(list(c.centroids), np.float32)[: 2 ** bits]
    got_m = np.array(list(c.midpoints), np.float32)[: 2 ** bits - 1]
    assert np.array_equal(got_c.view(np.uint32), c32.view(np.uint32))
    assert np.array_equal(got_m.view(np.uint32), m32.view(np.uint32))


@pytest.mark.parametrize("seed,layer", [(42, 0), (42, 7), (0, 3), (2 ** 40 + 5, 1)])
def test_layer_signs_equal_oracle(seed, layer):
    c = tq.config_init(128, 3, 4, True, seed)
    assert np.array_equal(tq.layer_signs(c, layer), OR.signs(seed, layer, 128))


def test_unknown_preset_error_text():
    with pytest.raises(tq.TQError) as ei:
        tq.config_from_preset("turboquant_2bit", 128)
    assert ei.value.status == 2
    assert ei.value.message == ("Unknown TurboQuant cache dtype: 'turboquant_2bit'. Valid presets: "
                                "turboquant_k8v4, turboquant_4bit_nc, turboquant_k3v4_nc, turboquant_3bit_nc")


@pytest.mark.parametrize("args,status", [((100, 3, 4), 3), ((128, 5, 4), 1), ((128, 3, 1), 1), ((128, 3, 5), 1),
                                         ((256, 3, 4), 3)])
def test_config_init_rejects(args, status):
    with pytest.raises(tq.TQError) as ei:
        tq.config_init(*args)
    assert ei.value.status == status


def _c_call(name, *args):
    return getattr(tq.lib(), name)(*args)


def test_quantize_argument_errors_before_launch():
    c = tq.config_from_preset("turboquant_4bit_nc", 128)
    buf = ctypes.create_string_buffer(4096 + 16)
    al = (ctypes.addressof(buf) + 15) & ~15
    cfgp = ctypes.byref(c)
    # NULL k
    assert _c_call("tq_quantize_append", cfgp, 0, None, al, 1, 4, 8, 1024, 1024, al, al, 10, 16, None) == 1
    # misaligned pool
    assert _c_call("tq_quantize_append", cfgp, 0, al, al, 1, 4, 8, 1024, 1024, al, al + 2, 10, 16, None) == 1
    # token stride too small
    assert _c_call("tq_quantize_append", cfgp, 0, al, al, 1, 4, 8, 512, 1024, al, al, 10, 16, None) == 1
    # bad dtype
    assert _c_call("tq_quantize_append", cfgp, 0, al, al, 7, 4, 8, 1024, 1024, al, al, 10, 16, None) == 1
    assert "dtype" in tq.last_error()
    # more KV heads than the launch grid takes
    assert _c_call("tq_quantize_append", cfgp, 0, al, al, 1, 4, 65536, 1 << 24, 1 << 24, al, al, 10, 16, None) == 3
    assert "65535" in tq.last_error()
    # zero tokens is a no-op success even with NULL pointers
    assert _c_call("tq_quantize_append", cfgp, 0, None, None, 1, 0, 8, 1024, 1024, None, None, 10, 16, None) == 0
    # a modified config is rejected
    bad = tq.config_from_preset("turboquant_4bit_nc", 128)
    bad.slot_size_aligned = 100
    assert _c_call("tq_quantize_append", ctypes.byref(bad), 0, al, al, 1, 4, 8, 1024, 1024, al, al, 10, 16, None) == 1


@pytest.mark.parametrize("preset,d", [("turboquant_4bit_nc", 128), ("turboquant_3bit_nc", 96), ("turboquant_k3v4_nc", 64)])
def test_midpoints_that_share_an_index_bin_are_refused(preset, d):
    """The Lloyd-Max index is read from equal bins holding at most one
    midpoint each: two midpoints edited to within a bin of each other make
    both append entry points refuse the config before any launch."""
    buf = ctypes.create_string_buffer(4096 + 16)
    al = (ctypes.addressof(buf) + 15) & ~15
    c = tq.config_from_preset(preset, d)
    nm = c.n_centroids - 1
    span = c.midpoints[nm - 1] - c.midpoints[0]
    k = nm // 2
    c.midpoints[k + 1] = c.midpoints[k] + span / 1000.0
    assert _c_call("tq_quantize_append", ctypes.byref(c), 0, al, al, 1, 4, 8, 1024, 1024, al, al, 10, 16, None) == 3
    assert "bins" in tq.last_error()
    assert _c_call("tq_ring_flush", ctypes.byref(c), 0, al, al, 128, al, al, al, 4, 2, 8, al, 10, 16, None) == 3
    assert "bins" in tq.last_error()


def _decode(c, **kw):
    buf = ctypes.create_string_buffer(1 << 16)
    al = (ctypes.addressof(buf) + 15) & ~15
    a = dict(q=al, qd=1, batch=2, hq=8, hkv=2, pool=al, nblocks=4, bs=16, tables=al, maxb=2, lens=al,
             maxlen=32, rk=None, rv=None, rl=None, rcap=0, scale=0.0, out=al, ws=al, wsb=1 << 15, split=0)
    a.update(kw)
    return _c_call("tq_decode_attention", ctypes.byref(c), 0, a["q"], a["qd"], a["batch"], a["hq"], a["hkv"],
                   a["pool"], a["nblocks"], a["bs"], a["tables"], a["maxb"], a["lens"], a["maxlen"], a["rk"],
                   a["rv"], a["rl"], a["rcap"], ctypes.c_float(a["scale"]), a["out"], a["ws"],
                   ctypes.c_size_t(a["wsb"]), a["split"], None)


def test_decode_argument_errors_before_launch():
    c = tq.config_from_preset("turboquant_3bit_nc", 128)
    assert _decode(c, hq=7) == 1                       # Hq not a multiple of Hkv
    assert _decode(c, hq=64, hkv=2) == 3               # more than 16 q heads per kv head
    assert _decode(c, bs=8) == 3                       # block size not a multiple of 16
    assert _decode(c, wsb=8) == 4 and "workspace" in tq.last_error()
    assert _decode(c, ws=None) == 4
    assert _decode(c, rcap=128) == 1                   # ring_cap without ring tensors
    assert _decode(c, rk=1024, rv=None) == 1           # half a ring
    assert _decode(c, split=24) == 1                   # split not a multiple of 16
    assert _decode(c, q=None) == 1
    assert _decode(c, batch=0) == 0                    # nothing to do
    assert _decode(c, batch=9000) == 3                 # batch above the work-list limit
    # one pool block of 2 GiB or more (2 heads x 2^24 tokens x 102 bytes)
    assert _decode(c, bs=1 << 24) == 3 and "2 GiB" in tq.last_error()
    assert _decode(c, bs=1 << 20, ws=None) == 4        # 214 MB blocks pass that check


def test_workspace_size_and_plan():
    c = tq.config_from_preset("turboquant_k8v4", 128)
    row = 132 * 4                                   # [m, l, -, -, acc[128]] fp32
    # 16 sequences x 8192 tokens, ranges of >= 256 tokens: at most
    # 16 * 32 * 512 / 16 wave rows + 16 * 32 segment rows of one query head
    b, n = tq.decode_workspace_size(c, 16, 32, 8192, 0, 256)
    assert n == 33 and b == 256 + (16384 + 512) * row
    # one ring partial per (sequence, query head) and 32 ring tokens
    b, n = tq.decode_workspace_size(c, 16, 32, 8192, 128, 256)
    assert n == 37 and b == 256 + (16384 + 512) * row + 16 * 32 * 4 * row
    _, n = tq.decode_workspace_size(c, 16, 32, 8192, 100, 256)
    assert n == 37
    b, n = tq.decode_workspace_size(c, 4, 8, 0, 0, 0)
    assert n == 0 and b == 256
    # automatic ranges: 512 tokens with FP8 keys, 256 with MSE keys
    _, n_auto = tq.decode_workspace_size(c, 16, 32, 8192)
    assert n_auto == 17
    _, n_auto = tq.decode_workspace_size(tq.config_from_preset("turboquant_4bit_nc", 128), 16, 32, 8192)
    assert n_auto == 33
    # the header grows with the batch (tile prefix per sequence); 100 tokens
    # are 7 tiles, 512-token ranges 32 tiles: ceil(100 * 8 * 7 / 32) = 175
    # wave rows + 800 segment rows, the block rounded up to 256 bytes
    b, _ = tq.decode_workspace_size(c, 100, 8, 100, 0, 0)
    assert b == 512 + -(-(975 * row) // 256) * 256


def test_prefill_workspace_size_and_errors():
    """One partial of D + 4 floats per (row, history split); rows padded to
    blocks of 32 per KV head, splits chosen for about 2048 waves with at
    least 1024 history tokens each."""
    c = tq.config_from_preset("turboquant_4bit_nc", 128)
    row = 132 * 4
    # 4 sequences, 8 KV heads, 512-token chunks of 4 query heads per KV head:
    # 2048 rows = 64 blocks per KV head, 2048 waves without a split
    assert tq.prefill_workspace_size(c, 4, 32, 8, 512, 32768, 2048) == 4 * 8 * 2048 * row
    # one sequence, 100-token chunk of 1 head: 4 blocks of 32 rows, 8 KV heads
    # = 32 waves; 64 ranges wanted, 10000 // 1024 = 9 allowed, ceil(10000 / 9)
    # -> 1120 tokens per range, 9 ranges
    assert tq.prefill_workspace_size(c, 1, 8, 8, 100, 10000, 1000) == 8 * 128 * 9 * row
    # no history: one split; 7 tokens x 8 heads = 56 rows, 2 blocks of 32
    assert tq.prefill_workspace_size(c, 2, 16, 2, 7, 0, 0) == 2 * 2 * 64 * row
    d96 = tq.config_from_preset("turboquant_k3v4_nc", 96)
    assert tq.prefill_workspace_size(d96, 1, 16, 2, 9, 0, 0) == 2 * 96 * 100 * 4
    buf = ctypes.create_string_buffer(4096 + 256)
    al = (ctypes.addressof(buf) + 255) & ~255
    cfgp = ctypes.byref(c)

    def call(max_chunk=4, hq=8, hkv=2, nblocks=1, max_hist=16, ws=4096, bs=16):
        return _c_call("tq_prefill_attention", cfgp, 0, al, tq.BF16, al, al, al, 1, max_chunk, hq, hkv, al, nblocks,
                       bs, al, 1, al, max_hist, ctypes.c_float(0.0), al, al, ws, None)

    assert call(hq=7) == 1                             # not a multiple of the KV heads
    assert call(bs=24) == 3                            # block size not a multiple of 16
    assert call(nblocks=0) == 1 and "one block" in tq.last_error()
    assert call(max_chunk=1 << 30, hq=16, hkv=1) == 3  # rows beyond 31 bits
    assert call(ws=16) == 4                            # workspace too small
    assert call(max_chunk=0) == 0                      # nothing to do


@pytest.mark.parametrize("num_layers", [0, 1, 2, 3, 4, 5, 10, 28, 32, 61])
@pytest.mark.parametrize("n", [-1, 0, 1, 2, 3, 40])
def test_boundary_skip_layers_match_oracle(num_layers, n):
    from oracle import cache as OCache
    assert tq.boundary_skip_layers(num_layers, n) == OCache.boundary_skip_layers(num_layers, n)
    assert tq.boundary_skip_layers(num_layers, n, hybrid=True) == []


@pytest.mark.parametrize("preset", PRESETS)
@pytest.mark.parametrize("d,hkv", [(64, 2), (96, 4), (128, 8)])
@pytest.mark.parametrize("skip_bytes", [0, 1, 2, 4])
def test_attn_page_size_matches_oracle(preset, d, hkv, skip_bytes):
    from oracle import cache as OCache
    assert tq.attn_page_size_1_token(tq.config_from_preset(preset, d), hkv, skip_bytes) == \
        OCache.attn_page_bytes_1_token(OC.from_cache_dtype(preset, d), hkv, skip_bytes)


def test_ring_argument_errors_before_launch():
    c = tq.config_from_preset("turboquant_3bit_nc", 128)
    buf = ctypes.create_string_buffer(4096 + 16)
    al = (ctypes.addressof(buf) + 15) & ~15
    cfgp = ctypes.byref(c)
    # flush: ring_cap 0, NULL ring_lens, misaligned pool; batch 0 is a no-op
    assert _c_call("tq_ring_flush", cfgp, 0, al, al, 0, al, al, al, 4, 2, 8, al, 10, 16, None) == 1
    assert _c_call("tq_ring_flush", cfgp, 0, al, al, 128, None, al, al, 4, 2, 8, al, 10, 16, None) == 1
    assert _c_call("tq_ring_flush", cfgp, 0, al, al, 128, al, al, al, 4, 2, 8, al + 2, 10, 16, None) == 1
    assert _c_call("tq_ring_flush", cfgp, 0, None, None, 128, None, None, None, 4, 0, 8, None, 10, 16, None) == 0
    # append: NULL k_new, misaligned ring; batch 0 is a no-op
    assert _c_call("tq_ring_append", cfgp, None, al, 2, 8, al, al, 128, al, None) == 1
    assert _c_call("tq_ring_append", cfgp, al, al, 2, 8, al + 4, al, 128, al, None) == 1
    assert _c_call("tq_ring_append", cfgp, None, None, 0, 8, None, None, 128, None, None) == 0


def test_check_slot_mapping():
    """The host debug check of a slot mapping: -1 skips, range, repeats."""
    tq.check_slot_mapping(np.array([0, 5, -1, 63, -1, 17], np.int64), 4, 16)   # 64 slots
    tq.check_slot_mapping(np.zeros(0, np.int64), 0, 16)
    for bad, idx in (([0, 64, 3], 1), ([3, -2], 1), ([7, 8, 9, 8, 7], 3), ([1, 1], 1)):
        with pytest.raises(tq.TQError) as ei:
            tq.check_slot_mapping(np.array(bad, np.int64), 4, 16)
        assert ei.value.status == tq.TQ_ERR_INVALID_ARG and ei.value.index == idx, (bad, ei.value.index)
    # the message names the two tokens of a repeated slot
    with pytest.raises(tq.TQError, match="tokens 0 and 3 both write slot 7"):
        tq.check_slot_mapping(np.array([7, 1, 2, 7], np.int64), 4, 16)
    # raw C-ABI: argument errors, NULL out-parameter
    lib = tq.lib()
    assert lib.tq_check_slot_mapping(None, 3, 4, 16, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_check_slot_mapping(None, 0, 4, 0, None) == tq.TQ_ERR_INVALID_ARG
    m = np.array([1, 2, 2], np.int64)
    assert lib.tq_check_slot_mapping(m.ctypes.data, 3, 4, 16, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_check_slot_mapping(m.ctypes.data, 2, 4, 16, None) == tq.TQ_OK


def test_check_block_tables():
    """The host debug check of block tables against lengths and the pool."""
    tables = np.array([[3, 0, 9], [1, -1, -1]], np.int32)
    tq.check_block_tables(tables, np.array([40, 16], np.int32), 10, 16)     # 3 and 1 blocks used
    tq.check_block_tables(tables, np.array([0, 0], np.int32), 10, 16)
    cases = [
        (np.array([[3, 0, 10], [1, 0, 0]], np.int32), [40, 16], (0, 2)),   # id past the pool
        (np.array([[3, 0, 9], [1, -1, 0]], np.int32), [40, 17], (1, 1)),   # negative id in use
        (tables, [49, 16], (0, -1)),                                       # 4 blocks, row of 3
        (tables, [40, -1], (1, -1)),                                       # negative length
    ]
    for t, lens, where in cases:
        with pytest.raises(tq.TQError) as ei:
            tq.check_block_tables(t, np.array(lens, np.int32), 10, 16)
        assert ei.value.status == tq.TQ_ERR_INVALID_ARG and (ei.value.seq, ei.value.block) == where, (lens, where)
    lib = tq.lib()
    assert lib.tq_check_block_tables(None, 1, 3, None, 10, 16, None, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_check_block_tables(None, 0, 3, None, 10, 16, None, None) == tq.TQ_OK
