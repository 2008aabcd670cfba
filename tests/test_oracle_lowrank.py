"""Pins of the oracle's low-rank correction (orka README, CLI: the correct
command adds a low-rank/sparse correction; the form U V added to the decoded
weight is this library's reading): a hand-computed fixture, a rank-one unit
case, the stated order of the float64 additions, the factor-wise error
scale, and the byte count."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def hand():
    with open(os.path.join(GOLDEN, "lowrank_hand.json")) as f:
        return json.load(f)


def hand_weight(c):
    cb = np.zeros((256, 8), np.float16)
    cb[0] = np.array(c["codebook_entry0"], np.float16)
    idx = [np.zeros(c["n_out"] * c["k_in"] // 8, np.int64)]
    scales = np.full((c["n_out"], 1), c["scale"], np.float16)
    lr = (np.array(c["U"], np.float16), np.array(c["V"], np.float16))
    return idx, [cb], scales, lr


def test_hand_fixture():
    c = hand()
    idx, cbs, scales, lr = hand_weight(c)
    n, k = c["n_out"], c["k_in"]
    plain = oracle.dequant_exact(n, k, idx, cbs, scales, k)
    assert np.array_equal(plain, np.tile(c["decoded_row"], (n, 1)))
    assert np.array_equal(oracle.lowrank_dense(n, k, lr), np.array(c["UV"]))
    w = oracle.dequant_exact(n, k, idx, cbs, scales, k, lowrank=lr)
    assert np.array_equal(w, np.array(c["W_eff"]))
    y, _ = oracle.matmul_ref(w, np.array(c["x"]))
    assert np.array_equal(y[0], np.array(c["y"]))
    assert np.array_equal(oracle.lowrank_bound(np.array(c["x"]), lr)[0], np.array(c["lowrank_bound_for_x"]))
    w16 = oracle.dequant_fp16(n, k, idx, cbs, scales, k, lowrank=lr)
    assert np.array_equal(w16.astype(np.float64), np.array(c["W_eff"]))


def test_rank_one_unit_row():
    """U = e_i (one column): only row i changes, by exactly V's row."""
    rng = np.random.default_rng(3)
    n, k = 5, 16
    u = np.zeros((n, 1), np.float16)
    u[3, 0] = 1.0
    v = rng.standard_normal((1, k)).astype(np.float16)
    d = oracle.lowrank_dense(n, k, (u, v))
    assert not d[[0, 1, 2, 4]].any()
    assert np.array_equal(d[3], v[0].astype(np.float64))


def test_dense_matches_matrix_product():
    """With small dyadic factors every sum is exact, so U V equals the
    library matrix product."""
    rng = np.random.default_rng(4)
    u = (rng.integers(-8, 9, (7, 4)) / 8.0).astype(np.float16)
    v = (rng.integers(-8, 9, (4, 24)) / 16.0).astype(np.float16)
    assert np.array_equal(oracle.lowrank_dense(7, 24, (u, v)), u.astype(np.float64) @ v.astype(np.float64))


def test_addition_order():
    """The rank-one terms are added to the decoded weight one at a time:
    2^30 + 2^-24 + 2^-24 + 2^-24 stays 2^30 (each term is a quarter ulp),
    while adding their sum 3 * 2^-24 (three quarters of an ulp) first would
    round up."""
    n, k = 1, 8
    cb = np.zeros((256, 8), np.float16)
    cb[0] = 2.0 ** 15
    scales = np.full((1, 1), 2.0 ** 15, np.float16)
    idx = [np.zeros(1, np.int64)]
    u = np.full((1, 3), 2.0 ** -12, np.float16)
    v = np.full((3, 8), 2.0 ** -12, np.float16)
    w = oracle.dequant_exact(n, k, idx, [cb], scales, k, lowrank=(u, v))
    assert np.all(w == 2.0 ** 30)
    assert 2.0 ** 30 + 3 * 2.0 ** -24 > 2.0 ** 30  # the other order differs


def test_bound_cancellation():
    """U V = 0 by cancellation, but the factor-wise scale keeps both terms."""
    u = np.array([[1.0, 1.0]], np.float16)
    v = np.array([[1.0, -2.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0], [-1.0, 2.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0]], np.float16)
    assert not oracle.lowrank_dense(1, 8, (u, v)).any()
    x = np.array([3.0, -1.0, 5, 5, 5, 5, 5, 5])
    assert oracle.lowrank_bound(x, (u, v))[0, 0] == 2 * (3 + 2)


def test_factor_shapes_checked():
    with pytest.raises(ValueError):
        oracle.lowrank_dense(2, 8, (np.zeros((2, 3)), np.zeros((2, 8))))
    with pytest.raises(ValueError):
        oracle.lowrank_dense(2, 8, (np.zeros((3, 2)), np.zeros((2, 8))))
    with pytest.raises(ValueError):
        oracle.lowrank_dense(2, 8, (np.zeros((2, 0)), np.zeros((0, 8))))


def test_bytes():
    base = oracle.compressed_bytes(4096, 4096, 2, 12, 128)
    assert oracle.compressed_bytes(4096, 4096, 2, 12, 128, lowrank_rank=16) == base + 2 * 16 * (4096 + 4096)
