"""Pins of the oracle's Lloyd-Max table against Max (1960) and the
optimality conditions, checked with independent scipy quadrature."""

import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import lloyd_max as LM
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "max1960_lloyd_max.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("levels", [4, 8, 16])
def test_matches_max_1960_table(levels):
    g = _golden()
    want = np.array(g["levels"][str(levels)]["outputs"])
    got = LM.standard_normal_table(levels)
    assert np.allclose(got[levels // 2:], want, atol=g["tolerance_outputs"])
    assert np.array_equal(got[: levels // 2], -got[levels // 2:][::-1])


def _mse(c):
    edges = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    total = 0.0
    for k in range(len(c)):
        val, _ = integrate.quad(lambda x: (x - c[k]) ** 2 * stats.norm.pdf(x), edges[k], edges[k + 1])
        total += val
    return total


@pytest.mark.parametrize("levels", [4, 8, 16])
def test_distortion_matches_max(levels):
    g = _golden()
    want = g["levels"][str(levels)]["mse"]
    got = _mse(LM.standard_normal_table(levels))
    assert abs(got - want) / want < g["tolerance_mse_relative"]


@pytest.mark.parametrize("levels", [4, 8, 16])
def test_centroid_condition(levels):
    c = LM.standard_normal_table(levels)
    edges = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    for k in range(levels):
        num, _ = integrate.quad(lambda x: x * stats.norm.pdf(x), edges[k], edges[k + 1], epsabs=1e-14)
        den = stats.norm.cdf(edges[k + 1]) - stats.norm.cdf(edges[k])
        assert abs(num / den - c[k]) < 1e-9


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fp32_tables(d, bits):
    c64 = LM.centroids_f64(d, bits)
    assert np.allclose(c64 * math.sqrt(d), LM.standard_normal_table(2 ** bits), rtol=1e-15)
    c32, m32 = LM.tables_f32(d, bits)
    assert c32.dtype == np.float32 and m32.dtype == np.float32
    assert len(c32) == 2 ** bits and len(m32) == 2 ** bits - 1
    # exact antisymmetry survives the fp32 rounding
    assert np.array_equal(c32, -c32[::-1])
    assert np.array_equal(m32, -m32[::-1])
    assert m32[len(m32) // 2] == 0.0
    # midpoint condition: each threshold is the (rounded) mean of its neighbours
    assert np.array_equal(m32, ((c64[:-1] + c64[1:]) / 2).astype(np.float32))
    assert np.all(np.diff(c32) > 0) and np.all((c32[:-1] < m32) & (m32 < c32[1:]))
