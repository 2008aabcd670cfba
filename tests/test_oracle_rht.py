"""Pins for the oracle's randomized Hadamard transform (GLQ page, "How it
works": sign flips then a fast Walsh-Hadamard transform; "Bit widths":
block-diagonal power-of-two decomposition)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from conftest import GOLDEN


@pytest.mark.parametrize("m", range(0, 11))
def test_fwht_equals_sylvester_matrix(m):
    """scipy.linalg.hadamard builds the Sylvester-order Hadamard matrix
    independently; the fast transform must equal it scaled by 1/sqrt(n)."""
    n = 1 << m
    rng = np.random.default_rng(m)
    v = rng.standard_normal(n)
    dense = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    assert np.allclose(oracle.fwht(v), dense @ v, rtol=0, atol=1e-12 * max(1.0, np.abs(v).sum()))


def test_fwht_small_closed_forms():
    a, b = 3.0, -5.0
    assert np.allclose(oracle.fwht([a, b]), [(a + b) / math.sqrt(2), (a - b) / math.sqrt(2)], atol=1e-15)
    assert oracle.fwht([7.5]).tolist() == [7.5]
    n = 256
    e0 = np.zeros(n)
    e0[0] = 1.0
    assert np.allclose(oracle.fwht(e0), np.full(n, 1 / math.sqrt(n)), atol=1e-15)
    # the last basis vector maps to the last Sylvester row: signs (-1)^popcount(i)
    el = np.zeros(n)
    el[-1] = 1.0
    want = np.array([(-1) ** bin(i).count("1") for i in range(n)]) / math.sqrt(n)
    assert np.allclose(oracle.fwht(el), want, atol=1e-15)


def test_fwht_involution_and_parseval():
    rng = np.random.default_rng(5)
    for n in (1, 2, 64, 8192):
        v = rng.standard_normal(n)
        t = oracle.fwht(v)
        assert abs(np.linalg.norm(t) - np.linalg.norm(v)) <= 1e-12 * np.linalg.norm(v)
        assert np.allclose(oracle.fwht(t), v, atol=1e-12)


def test_fwht_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.fwht(np.zeros(12))


def _block_cases():
    with open(os.path.join(GOLDEN, "rht_blocks.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _block_cases(), ids=lambda c: f"{c['n']}/{c['max_block']}")
def test_block_decomposition(case):
    assert oracle.rht_blocks(case["n"], case["max_block"]) == case["blocks"]


def test_rht_equals_block_diagonal_dense():
    """x' = blockdiag(H_n1/sqrt(n1), ...) (sigma * x), built densely with scipy."""
    rng = np.random.default_rng(8)
    n = 2688
    signs = rng.integers(0, 2, n) * 2 - 1
    x = rng.standard_normal((3, n))
    blocks = oracle.rht_blocks(n, 8192)
    dense = scipy.linalg.block_diag(*[scipy.linalg.hadamard(b) / math.sqrt(b) for b in blocks])
    got = oracle.rht_ref(x, signs, 8192)
    want = (dense @ (x * signs).T).T
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(x).sum())


def test_rht_signs_first():
    """Signs act before the transform: with x = e_0 and sigma_0 = -1 the first
    block is -1/sqrt(n) everywhere (a transform-then-sign reading would give
    only the first entry negative)."""
    n = 64
    signs = np.ones(n)
    signs[0] = -1
    x = np.zeros(n)
    x[0] = 1.0
    got = oracle.rht_ref(x, signs, 64)[0]
    assert np.allclose(got, -np.ones(n) / 8.0, atol=1e-15)


def test_rht_preserves_norm_per_block():
    rng = np.random.default_rng(9)
    n = 28672
    signs = rng.integers(0, 2, n) * 2 - 1
    x = rng.standard_normal(n)
    got = oracle.rht_ref(x, signs, 8192)[0]
    off = 0
    for b in oracle.rht_blocks(n, 8192):
        assert abs(np.linalg.norm(got[off:off + b]) - np.linalg.norm(x[off:off + b])) <= 1e-10
        off += b


def test_inverse_is_dense_transpose():
    """The output transform is (H D)^T = D H, built densely with scipy: the
    transpose of the input transform's matrix."""
    rng = np.random.default_rng(10)
    n = 2688
    signs = rng.integers(0, 2, n) * 2 - 1
    y = rng.standard_normal((2, n))
    blocks = oracle.rht_blocks(n, 1024)
    fwd = scipy.linalg.block_diag(*[scipy.linalg.hadamard(b) / math.sqrt(b) for b in blocks]) @ np.diag(signs)
    got = oracle.rht_inverse_ref(y, signs, 1024)
    want = (fwd.T @ y.T).T
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(y).sum())


def test_inverse_signs_last():
    """Signs act after the transform: with y = e_0 and sigma_0 = -1 only the
    first output is negative (a sign-first reading would negate them all)."""
    n = 64
    signs = np.ones(n)
    signs[0] = -1
    y = np.zeros(n)
    y[0] = 1.0
    got = oracle.rht_inverse_ref(y, signs, 64)[0]
    want = np.ones(n) / 8.0
    want[0] = -1 / 8.0
    assert np.allclose(got, want, atol=1e-15)


@pytest.mark.parametrize("n,mb", [(28672, 8192), (2688, 8192), (576, 64), (1, 1)])
def test_inverse_round_trip(n, mb):
    rng = np.random.default_rng(n)
    signs = rng.integers(0, 2, n) * 2 - 1
    x = rng.standard_normal((2, n))
    back = oracle.rht_inverse_ref(oracle.rht_ref(x, signs, mb), signs, mb)
    assert np.allclose(back, x, rtol=0, atol=1e-12 * np.sqrt(n))


def test_shards_dense():
    """Shards 12 | 8 with blocks of at most 8: blockdiag(H8, H4 | H8), each
    shard's decomposition restarting at its own boundary (one decomposition
    of the whole row of 20 would give H16, H4 instead)."""
    rng = np.random.default_rng(11)
    signs = rng.integers(0, 2, 20) * 2 - 1
    x = rng.standard_normal((3, 20))
    h = [scipy.linalg.hadamard(b) / math.sqrt(b) for b in (8, 4, 8)]
    dense = scipy.linalg.block_diag(*h)
    got = oracle.rht_shards_ref(x, [12, 8], signs, 8)
    assert np.allclose(got, (dense @ (x * signs).T).T, rtol=0, atol=1e-13)
    got_inv = oracle.rht_shards_ref(x, [12, 8], signs, 8, inverse=True)
    assert np.allclose(got_inv, ((dense @ x.T).T) * signs, rtol=0, atol=1e-13)
    whole = oracle.rht_ref(x, signs, 16)
    assert not np.allclose(oracle.rht_shards_ref(x, [12, 8], signs, 16), whole)


def test_shards_reject_bad_lengths():
    with pytest.raises(ValueError):
        oracle.rht_shards_ref(np.zeros((1, 8)), [4, 3], np.ones(8), 8)
    with pytest.raises(ValueError):
        oracle.rht_shards_ref(np.zeros((1, 8)), [8, 0], np.ones(8), 8)
