"""Pins for the oracle's matmul Y = X dequant(W)^T (GLQ page, "Inference
kernels") and its acceptance bound."""
from fractions import Fraction

import numpy as np

import oracle


def _rand_weight(rng, n, k, stages=2, bits=12, bs=128, sd=(0.02, 0.006)):
    cbs = [(rng.standard_normal((1 << bits, 8)) * sd[t]).astype(np.float16) for t in range(stages)]
    idx = [rng.integers(0, 1 << bits, n * k // 8) for _ in range(stages)]
    sc = rng.uniform(0.5, 1.5, (n, oracle.n_scale_blocks(k, bs))).astype(np.float16)
    return cbs, idx, sc


def test_one_hot_recovers_dequantized_columns():
    rng = np.random.default_rng(1)
    n, k = 24, 96
    cbs, idx, sc = _rand_weight(rng, n, k, bs=32)
    w64 = oracle.dequant_exact(n, k, idx, cbs, sc, 32)
    for col in (0, 7, 8, 31, 32, 95):
        x = np.zeros((1, k))
        x[0, col] = 1.0
        y, bound = oracle.matmul_ref(w64, x)
        assert np.array_equal(y[0], w64[:, col])
        assert np.array_equal(bound[0], np.abs(w64[:, col]))


def test_zero_codebook_gives_zero():
    rng = np.random.default_rng(2)
    n, k = 8, 64
    cbs = [np.zeros((256, 8), np.float16)]
    idx = [rng.integers(0, 256, n * k // 8)]
    sc = rng.uniform(0.5, 1.5, (n, 1)).astype(np.float16)
    w64 = oracle.dequant_exact(n, k, idx, cbs, sc, k)
    y, _ = oracle.matmul_ref(w64, rng.standard_normal((3, k)))
    assert np.all(y == 0.0)


def test_single_entry_codebook_closed_form():
    """All indices 0 and cb[0] = v: y_r = sum_g s[r, blk(g)] <v, x_g>."""
    rng = np.random.default_rng(4)
    n, k, bs = 6, 80, 16
    v = (rng.standard_normal(8) * 0.1).astype(np.float16)
    cb = np.zeros((16, 8), np.float16)
    cb[0] = v
    idx = [np.zeros(n * k // 8, dtype=np.int64)]
    sc = rng.uniform(0.5, 1.5, (n, oracle.n_scale_blocks(k, bs))).astype(np.float16)
    x = rng.standard_normal(k)
    w64 = oracle.dequant_exact(n, k, idx, [cb], sc, bs)
    y, _ = oracle.matmul_ref(w64, x)
    v64 = v.astype(np.float64)
    for r in range(n):
        want = sum(float(sc[r, (8 * g) // bs]) * float(v64 @ x[8 * g:8 * g + 8]) for g in range(k // 8))
        assert abs(y[0, r] - want) <= 1e-12 * (1 + abs(want))


def test_fraction_brute_force_tiny():
    """Exact rational Y for a tiny 2-stage weight and 2 tokens agrees with the
    float64 oracle to float64 rounding (relative to the bound)."""
    rng = np.random.default_rng(9)
    n, k = 4, 32
    cbs, idx, sc = _rand_weight(rng, n, k, bs=16)
    x = rng.standard_normal((2, k)).astype(np.float32)
    w64 = oracle.dequant_exact(n, k, idx, cbs, sc, 16)
    y, bound = oracle.matmul_ref(w64, x)
    for b in range(2):
        for r in range(n):
            exact = Fraction(0)
            tot = Fraction(0)
            for c in range(k):
                f = r * (k // 8) + c // 8
                wv = Fraction(float(sc[r, c // 16])) * (Fraction(float(cbs[0][idx[0][f], c % 8])) +
                                                      Fraction(float(cbs[1][idx[1][f], c % 8])))
                exact += wv * Fraction(float(x[b, c]))
                tot += abs(wv * Fraction(float(x[b, c])))
            assert abs(Fraction(float(y[b, r])) - exact) <= Fraction(1, 2 ** 45) * tot
            assert abs(Fraction(float(bound[b, r])) - tot) <= Fraction(1, 2 ** 45) * tot


def test_naive_triple_loop():
    rng = np.random.default_rng(10)
    n, k, b = 5, 24, 3
    cbs, idx, sc = _rand_weight(rng, n, k, stages=1, bits=8, bs=8)
    w64 = oracle.dequant_exact(n, k, idx, cbs, sc, 8)
    x = rng.standard_normal((b, k))
    y, bound = oracle.matmul_ref(w64, x)
    for i in range(b):
        for r in range(n):
            acc = 0.0
            for c in range(k):
                acc += w64[r, c] * x[i, c]
            assert abs(acc - y[i, r]) <= 1e-12 * bound[i, r]


def test_linearity():
    rng = np.random.default_rng(12)
    n, k = 7, 64
    cbs, idx, sc = _rand_weight(rng, n, k, bs=64)
    w64 = oracle.dequant_exact(n, k, idx, cbs, sc, 64)
    x1, x2 = rng.standard_normal((2, k))
    y1, b1 = oracle.matmul_ref(w64, x1)
    y2, b2 = oracle.matmul_ref(w64, x2)
    y3, _ = oracle.matmul_ref(w64, 2.0 * x1 - 3.0 * x2)
    assert np.all(np.abs(y3 - (2 * y1 - 3 * y2)) <= 1e-12 * (2 * b1 + 3 * b2))


def test_tolerance_predicate():
    y_ref = np.array([1.0, -2.0, 0.0])
    bound = np.array([10.0, 100.0, 0.0])
    ok, worst = oracle.within_tolerance(y_ref + np.array([0.02, -0.2, 1e-6]), y_ref, bound)
    assert ok.all() and abs(worst - 1.0) < 1e-9
    ok, _ = oracle.within_tolerance(y_ref + np.array([0.0201, 0.0, 0.0]), y_ref, bound)
    assert not ok[0] and ok[1:].all()


def test_one_hot_recovers_corrected_column():
    """One-hot x = e_k picks column k of the decoded weight plus its sparse
    correction exactly."""
    rng = np.random.default_rng(33)
    n, k = 9, 40
    cb = [(rng.standard_normal((256, 8)) * 0.02).astype(np.float16)]
    idx = [rng.integers(0, 256, n * k // 8)]
    sc = rng.uniform(0.5, 1.5, (n, 5)).astype(np.float16)
    rowptr = np.array([0, 1, 1, 3, 3, 3, 4, 4, 4, 6])
    col = np.array([7, 7, 7, 39, 0, 7])
    val = np.array([0.5, -0.25, 0.125, 1.0, 2.0, -1.0], np.float16)
    w64 = oracle.dequant_exact(n, k, idx, cb, sc, 8, sparse=(rowptr, col, val))
    plain = oracle.dequant_exact(n, k, idx, cb, sc, 8)
    x = np.zeros((1, k))
    x[0, 7] = 1.0
    y, _ = oracle.matmul_ref(w64, x)
    assert np.array_equal(y[0], w64[:, 7])
    assert y[0, 0] == plain[0, 7] + 0.5 and y[0, 2] == plain[2, 7] + (-0.25 + 0.125) and y[0, 8] == plain[8, 7] - 1.0
    assert y[0, 1] == plain[1, 7]
