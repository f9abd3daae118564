"""Pins of the oracle's random signs and Walsh-Hadamard rotation."""

import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import config as C
from oracle import rotation as R
from tests.conftest import GOLDEN


def test_splitmix64_published_vectors():
    with open(os.path.join(GOLDEN, "splitmix64_vectors.json")) as f:
        data = json.load(f)
    for vec in data["vectors"]:
        want = [int(x) for x in vec["outputs"]]
        assert R.splitmix64(vec["seed"], len(want)) == want


def test_signs_per_layer_seed():
    # layer l uses base seed + 1337 l (TurboQuantConfig docstring, seed argument)
    for layer in (0, 1, 5):
        a = R.signs(42, layer, 128)
        b = R.signs(42 + 1337 * layer, 0, 128)
        assert np.array_equal(a, b)
    s = R.signs(42, 0, 128)
    assert set(np.unique(s)) <= {-1.0, 1.0}
    # a fair coin: 128 signs are not all equal and roughly balanced
    assert 32 < (s > 0).sum() < 96
    assert not np.array_equal(R.signs(42, 0, 128), R.signs(42, 1, 128))


def test_signs_are_top_bits():
    outs = R.splitmix64(7, 64)
    s = R.signs(7, 0, 64)
    for j, z in enumerate(outs):
        assert s[j] == (-1.0 if z >= 2 ** 63 else 1.0)


@pytest.mark.parametrize("block", [2, 4, 8, 32, 64, 128])
def test_butterfly_is_sylvester_hadamard(block):
    eye = np.eye(block)
    h = scipy.linalg.hadamard(block)
    # row i of the butterfly of e_i's is column i of H (H symmetric)
    assert np.array_equal(R.butterfly_f64(eye, block), h.T)
    assert np.array_equal(R.butterfly_f32(eye.astype(np.float32), block), h.T.astype(np.float32))


def test_blockwise_for_96():
    eye = np.eye(96)
    h = scipy.linalg.hadamard(32)
    want = scipy.linalg.block_diag(h, h, h)
    assert np.array_equal(R.butterfly_f64(eye, 32), want.T)


@pytest.mark.parametrize("d", [64, 96, 128])
def test_rotation_orthogonal_and_round_trip(d):
    blk = C.TQConfig(head_dim=d).wht_block
    s = R.signs(42, 2, d).astype(np.float64)
    pi = R.rotate_f64(np.eye(d), s, blk).T  # column j = Pi e_j
    assert np.allclose(pi @ pi.T, np.eye(d), atol=1e-12)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, d))
    y = R.rotate_f64(x, s, blk)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    assert np.allclose(R.unrotate_f64(y, s, blk), x, atol=1e-12)
    # matches the explicit matrix (1/sqrt B) H diag(s), blockwise
    h = scipy.linalg.hadamard(blk) / np.sqrt(blk)
    full = scipy.linalg.block_diag(*([h] * (d // blk))) @ np.diag(s)
    assert np.allclose(y, x @ full.T, atol=1e-12)


def test_butterfly_stage_order_irrelevant_in_exact_arithmetic():
    # integer inputs: every partial sum is exact, so any stage order gives H x
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1000, size=(3, 128)).astype(np.float64)
    h = scipy.linalg.hadamard(128)
    assert np.array_equal(R.butterfly_f64(x, 128), x @ h.T)
