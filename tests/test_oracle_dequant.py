"""Pins for the oracle's dequant (orka README, "How it works": scale x sum of
codebook entries) and its single rounding to fp16."""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def fraction_to_half_bits(q: Fraction) -> int:
    """Round an exact rational to IEEE binary16 (nearest, ties to even), by
    hand, independent of numpy.  Returns the 16-bit pattern."""
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sign
    # find e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)                      # subnormal range shares exponent -14
    ulp = Fraction(2) ** (e - 10)
    m = a / ulp                          # significand in units of ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n == 2048:                        # carried into the next binade
        n = 1024
        e += 1
    if e > 15:
        return sign | 0x7C00             # overflow -> inf
    if n < 1024:                         # subnormal (only when e == -14)
        return sign | n
    return sign | ((e + 15) << 10) | (n - 1024)


def test_hand_rounding_helper_matches_struct():
    """The hand rounding above agrees with Python's own half packing on a
    spread of exact float64 values (both are single roundings)."""
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000),
                           [65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 0.0]])
    for v in vals:
        want = struct.unpack("<H", struct.pack("<e", float(v)))[0] if abs(v) < 65520 else (0x7C00 | (0x8000 if v < 0 else 0))
        assert fraction_to_half_bits(Fraction(float(v))) == want, v


def _load_cases():
    with open(os.path.join(GOLDEN, "dequant_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_hand_groups(case):
    idx = [np.array(i) for i in case["indices"]]
    cbs = [np.array(cb, dtype=np.float16) for cb in case["codebooks"]]
    sc = np.array(case["scales"], dtype=np.float16)
    w = oracle.dequant_fp16(case["n_out"], case["k_in"], idx, cbs, sc, case["scale_block"])
    want = np.array(case["w"], dtype=np.float16)
    assert np.array_equal(w.view(np.uint16), want.view(np.uint16))
    w64 = oracle.dequant_exact(case["n_out"], case["k_in"], idx, cbs, sc, case["scale_block"])
    assert np.array_equal(w64, np.array(case["w"], dtype=np.float64))


def test_double_rounding_trap():
    with open(os.path.join(GOLDEN, "double_rounding.json")) as f:
        d = json.load(f)
    cb0 = np.zeros((2, 8), np.float16)
    cb1 = np.zeros((2, 8), np.float16)
    cb0[1, :] = d["c0"]
    cb1[1, :] = d["c1"]
    w = oracle.dequant_fp16(1, 8, [np.array([1]), np.array([1])], [cb0, cb1],
                            np.array([[d["scale"]]], np.float16), 8)
    assert int(w.view(np.uint16)[0, 0]) == d["w_fp16_bits"]
    # the trap is real: going through fp32 first gives the other neighbour
    exact = float(np.float16(d["scale"])) * (float(np.float16(d["c0"])) + float(np.float16(d["c1"])))
    assert int(np.float16(np.float32(exact)).view(np.uint16)) == d["double_rounded_bits"]


def test_fraction_brute_force_tiny():
    """Exact rational dequant of random tiny tensors, rounded by hand, equals
    the oracle bit for bit (N=4, K=32, 2 stages, 12-bit, 16-column blocks)."""
    rng = np.random.default_rng(123)
    n, k, bs = 4, 32, 16
    for trial in range(5):
        cbs = [(rng.standard_normal((4096, 8)) * sd).astype(np.float16) for sd in (0.02, 0.006)]
        idx = [rng.integers(0, 4096, n * k // 8) for _ in range(2)]
        sc = rng.uniform(0.5, 1.5, (n, 2)).astype(np.float16)
        w = oracle.dequant_fp16(n, k, idx, cbs, sc, bs)
        w64 = oracle.dequant_exact(n, k, idx, cbs, sc, bs)
        for r in range(n):
            for c in range(k):
                g = c // 8
                f = r * (k // 8) + g
                tot = Fraction(float(cbs[0][idx[0][f], c % 8])) + Fraction(float(cbs[1][idx[1][f], c % 8]))
                q = Fraction(float(sc[r, c // bs])) * tot
                assert Fraction(float(w64[r, c])) == q
                assert int(w.view(np.uint16)[r, c]) == fraction_to_half_bits(q)


def test_fraction_brute_force_extremes():
    """Values at the ends of the fp16 range: subnormal sums, overflow to inf,
    negative scales -- exact in float64 and rounded once."""
    rng = np.random.default_rng(7)
    pool = np.array([6e-8, -6e-8, 1.2e-7, 3.0e-5, -6.1e-5, 0.5, -1.0, 100.0, 30000.0, 65504.0, -65504.0],
                    dtype=np.float16)
    n, k = 3, 16
    for _ in range(20):
        cbs = [rng.choice(pool, (4, 8)).astype(np.float16) for _ in range(3)]
        idx = [rng.integers(0, 4, n * 2) for _ in range(3)]
        sc = rng.choice(np.array([0.5, -2.0, 1.5, 6e-8, 1024.0], np.float16), (n, 1)).astype(np.float16)
        with np.errstate(over="ignore"):
            w = oracle.dequant_fp16(n, k, idx, cbs, sc, 16)
        for r in range(n):
            for c in range(k):
                f = r * 2 + c // 8
                q = Fraction(float(sc[r, 0])) * sum(Fraction(float(cbs[t][idx[t][f], c % 8])) for t in range(3))
                assert int(w.view(np.uint16)[r, c]) == fraction_to_half_bits(q) or (q == 0 and w[r, c] == 0)


def test_scale_block_boundaries():
    """K=576 with 128-column blocks: 5 blocks, the last covering 64 columns;
    each column takes the scale of block floor(col/128)."""
    assert oracle.n_scale_blocks(576, 128) == 5
    assert oracle.n_scale_blocks(512, 128) == 4
    assert oracle.n_scale_blocks(8192, 8192) == 1
    n, k, bs = 2, 576, 128
    cb = np.ones((1, 8), np.float16)
    idx = [np.zeros(n * k // 8, dtype=np.int64)]
    sc = np.array([[1, 2, 4, 8, 16], [-1, -2, -4, -8, -16]], np.float16)
    w = oracle.dequant_exact(n, k, idx, [cb], sc, bs)
    for c in range(k):
        assert w[0, c] == 2.0 ** (c // 128)
        assert w[1, c] == -(2.0 ** (c // 128))


def test_residual_sum_matches_stagewise_sum():
    """Invariant: dequant of two stages = the two one-stage dequants added
    (exactly, for values whose sum is exact) -- catches a dropped stage."""
    rng = np.random.default_rng(3)
    n, k = 5, 64
    cbs = [(rng.standard_normal((256, 8)) * 0.02).astype(np.float16) for _ in range(2)]
    idx = [rng.integers(0, 256, n * k // 8) for _ in range(2)]
    sc = rng.uniform(0.5, 1.5, (n, 1)).astype(np.float16)
    both = oracle.dequant_exact(n, k, idx, cbs, sc, k)
    a = oracle.dequant_exact(n, k, idx[:1], cbs[:1], sc, k)
    b = oracle.dequant_exact(n, k, idx[1:], cbs[1:], sc, k)
    assert np.array_equal(both, a + b)


# ---------------------------------------------------------------------------
# residual ladders: per-stage widths and per-stage residual scales
# ---------------------------------------------------------------------------

def _stage_cases():
    with open(os.path.join(GOLDEN, "stage_scale_hand.json")) as f:
        return json.load(f)["cases"]


def _sparse_codebooks(case):
    cbs = []
    for spec in case["codebooks_sparse"]:
        cb = np.zeros((spec["rows"], 8), np.float16)
        for row, vals in spec["set"].items():
            cb[int(row)] = vals
        cbs.append(cb)
    return cbs


@pytest.mark.parametrize("case", _stage_cases(), ids=lambda c: c["name"])
def test_stage_scale_hand(case):
    idx = [np.array(i) for i in case["indices"]]
    cbs = _sparse_codebooks(case)
    sc = np.array(case["scales"], dtype=np.float16)
    rs = np.array(case["stage_scales"], dtype=np.float32)
    assert np.array_equal(rs.astype(np.float64), np.array(case["stage_scales"]))  # fp32-exact inputs
    w = oracle.dequant_fp16(case["n_out"], case["k_in"], idx, cbs, sc, case["scale_block"], stage_scales=rs)
    if "w" in case:
        want = np.array(case["w"], dtype=np.float16)
        assert np.array_equal(w.view(np.uint16), want.view(np.uint16))
        w64 = oracle.dequant_exact(case["n_out"], case["k_in"], idx, cbs, sc, case["scale_block"], rs)
        assert np.array_equal(np.signbit(w64), np.signbit(np.array(case["w"])))
        assert np.array_equal(w64, np.array(case["w"]))
    else:
        assert w.view(np.uint16).tolist() == case["w_bits"]
        # the tie is real: the exact rational value rounds to the other neighbour
        q = sum(Fraction(float(rs[t])) * Fraction(float(cbs[t][idx[t][0], 0])) for t in range(2))
        q *= Fraction(float(sc[0, 0]))
        assert fraction_to_half_bits(q) == case["exact_real_bits"]


def test_unit_stage_scales_change_nothing():
    """r_t = 1 for every stage gives the plain decode bit for bit (ladder of
    mixed widths, subnormal-heavy codebooks, negative scales)."""
    rng = np.random.default_rng(29)
    n, k, bs = 6, 64, 32
    widths = [16, 8, 4]
    cbs = [(rng.standard_normal((1 << b, 8)) * 10.0 ** rng.integers(-7, 1, (1 << b, 8))).astype(np.float16)
           for b in widths]
    idx = [rng.integers(0, 1 << b, n * k // 8) for b in widths]
    sc = rng.uniform(-1.5, 1.5, (n, 2)).astype(np.float16)
    a = oracle.dequant_exact(n, k, idx, cbs, sc, bs)
    b = oracle.dequant_exact(n, k, idx, cbs, sc, bs, stage_scales=np.ones(3, np.float32))
    assert np.array_equal(a, b) and np.array_equal(np.signbit(a), np.signbit(b))


def test_stage_scale_fraction_brute_force():
    """12+4 and 16+8 ladders with float32 residual scales on random tiny
    tensors: the oracle's fp16 equals the exact rational value rounded by
    hand (the float64 evaluation order only matters within 2^-50 of a tie,
    which random data does not reach), and its float64 value is within
    2^-50 relative of the exact one."""
    rng = np.random.default_rng(41)
    n, k, bs = 3, 32, 16
    for widths in ([12, 4], [16, 8], [8, 8, 4, 4]):
        for _ in range(3):
            cbs = [(rng.standard_normal((1 << b, 8)) * 0.02 * 0.3 ** t).astype(np.float16)
                   for t, b in enumerate(widths)]
            idx = [rng.integers(0, 1 << b, n * k // 8) for b in widths]
            sc = rng.uniform(0.5, 1.5, (n, 2)).astype(np.float16)
            rs = rng.uniform(-3.0, 3.0, len(widths)).astype(np.float32)
            w = oracle.dequant_fp16(n, k, idx, cbs, sc, bs, stage_scales=rs)
            w64 = oracle.dequant_exact(n, k, idx, cbs, sc, bs, stage_scales=rs)
            for r in range(n):
                for c in range(k):
                    f = r * (k // 8) + c // 8
                    tot = sum(Fraction(float(rs[t])) * Fraction(float(cbs[t][idx[t][f], c % 8]))
                              for t in range(len(widths)))
                    q = Fraction(float(sc[r, c // bs])) * tot
                    assert abs(Fraction(float(w64[r, c])) - q) <= abs(q) * Fraction(1, 2 ** 50)
                    assert int(w.view(np.uint16)[r, c]) == fraction_to_half_bits(q), (widths, r, c)


def test_stage_scales_validated():
    cb = [np.ones((16, 8), np.float16)] * 2
    idx = [np.zeros(1, np.int64)] * 2
    sc = np.ones((1, 1), np.float16)
    with pytest.raises(ValueError):
        oracle.dequant_exact(1, 8, idx, cb, sc, 8, stage_scales=[1.0])
    with pytest.raises(ValueError):
        oracle.dequant_exact(1, 8, idx, cb, sc, 8, stage_scales=[1.0, float("inf")])


# ---------------------------------------------------------------------------
# sparse correction
# ---------------------------------------------------------------------------

def _sparse_case():
    with open(os.path.join(GOLDEN, "sparse_hand.json")) as f:
        return json.load(f)["cases"][0]


def test_sparse_hand():
    c = _sparse_case()
    cb = np.array(c["codebook"], np.float16)
    sp = (np.array(c["rowptr"]), np.array(c["col"]), np.array(c["val"], np.float16))
    w = oracle.dequant_fp16(c["n_out"], c["k_in"], [np.array(c["indices"])], [cb],
                            np.array(c["scales"], np.float16), c["scale_block"], sparse=sp)
    want = np.array(c["w"], np.float16)
    assert np.array_equal(w.view(np.uint16), want.view(np.uint16))


def test_sparse_alone_and_linearity():
    """With an all-zero codebook the weight is the correction alone; in
    general the correction adds exactly (small dyadic-free values whose sums
    are exact in float64)."""
    rng = np.random.default_rng(8)
    n, k = 7, 64
    nnz_row = rng.integers(0, 6, n)
    rowptr = np.concatenate([[0], np.cumsum(nnz_row)])
    col = np.concatenate([np.sort(rng.choice(k, m, replace=False)) for m in nnz_row]).astype(np.int64)
    val = (rng.standard_normal(rowptr[-1]) * 0.1).astype(np.float16)
    sp = (rowptr, col, val)
    idx = [rng.integers(0, 256, n * k // 8)]
    sc = rng.uniform(0.5, 1.5, (n, 2)).astype(np.float16)
    zero = [np.zeros((256, 8), np.float16)]
    assert np.array_equal(oracle.dequant_exact(n, k, idx, zero, sc, 32, sparse=sp), oracle.sparse_dense(n, k, sp))
    cb = [(rng.standard_normal((256, 8)) * 0.02).astype(np.float16)]
    base = oracle.dequant_exact(n, k, idx, cb, sc, 32)
    withc = oracle.dequant_exact(n, k, idx, cb, sc, 32, sparse=sp)
    dense = oracle.sparse_dense(n, k, sp)
    assert np.allclose(withc, base + dense, rtol=0, atol=1e-15)
    assert np.array_equal(withc[dense == 0], base[dense == 0])
    empty = (np.zeros(n + 1, np.int64), np.zeros(0, np.int64), np.zeros(0, np.float16))
    assert np.array_equal(oracle.dequant_exact(n, k, idx, cb, sc, 32, sparse=empty), base)


def test_sparse_fraction_brute_force():
    """Exact rational decode + correction, rounded by hand, equals the oracle's
    fp16 (12+4 ladder with stage scales and a correction with repeated
    columns)."""
    rng = np.random.default_rng(21)
    n, k, bs = 3, 32, 16
    cbs = [(rng.standard_normal((1 << b, 8)) * 0.02).astype(np.float16) for b in (12, 4)]
    idx = [rng.integers(0, 1 << b, n * k // 8) for b in (12, 4)]
    sc = rng.uniform(0.5, 1.5, (n, 2)).astype(np.float16)
    rs = np.array([1.0, 0.3], np.float32)
    rowptr = np.array([0, 4, 4, 9])
    col = np.array([0, 5, 5, 31, 1, 2, 2, 2, 30])
    val = (rng.standard_normal(9) * 0.01).astype(np.float16)
    sp = (rowptr, col, val)
    w = oracle.dequant_fp16(n, k, idx, cbs, sc, bs, stage_scales=rs, sparse=sp)
    for r in range(n):
        for c in range(k):
            f = r * (k // 8) + c // 8
            q = Fraction(float(sc[r, c // bs])) * sum(Fraction(float(rs[t])) * Fraction(float(cbs[t][idx[t][f], c % 8]))
                                                     for t in range(2))
            q += sum(Fraction(float(val[j])) for j in range(rowptr[r], rowptr[r + 1]) if col[j] == c)
            assert int(w.view(np.uint16)[r, c]) == fraction_to_half_bits(q), (r, c)


def test_sparse_validated():
    cb = [np.ones((256, 8), np.float16)]
    idx = [np.zeros(2, np.int64)]
    sc = np.ones((1, 1), np.float16)
    for bad in [([0, 2], [0, 16], [1.0, 1.0]),       # column out of range
                ([1, 2], [0, 1], [1.0, 1.0]),        # rowptr[0] != 0
                ([0, 3], [0, 1], [1.0, 1.0]),        # too few entries
                ([0], [], [])]:                      # wrong rowptr length
        with pytest.raises(ValueError):
            oracle.dequant_exact(1, 16, idx, cb, sc, 16, sparse=tuple(np.array(v) for v in bad))
