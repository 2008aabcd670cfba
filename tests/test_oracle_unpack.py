"""Pins for the oracle's bit-plane unpack (orka README, "How it works")."""
import json
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "bitplane_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["note"][:24])
def test_hand_planes_unpack(case):
    """Planes worked by hand decode to the stated indices (no use of pack)."""
    lo = None if case["lo"] is None else np.array(case["lo"], dtype=np.uint8)
    hi = None if case["hi"] is None else np.array(case["hi"], dtype=np.uint8)
    got = oracle.unpack_indices(case["bits"], len(case["indices"]), lo=lo, hi=hi)
    assert got.tolist() == case["indices"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["note"][:24])
def test_hand_indices_pack(case):
    lo, hi = oracle.pack_indices(case["indices"], case["bits"])
    if case["lo"] is None:
        assert lo is None
    else:
        assert lo.tolist() == case["lo"]
    if case["hi"] is None:
        assert hi is None
    else:
        assert hi.tolist() == case["hi"]


def test_exhaustive_12bit_roundtrip():
    """Every 12-bit value survives pack -> unpack, at both nibble positions."""
    vals = np.arange(4096)
    for seq in (vals, vals[::-1], np.roll(vals, 1), vals[:4095]):
        lo, hi = oracle.pack_indices(seq, 12)
        assert lo.size == seq.size and hi.size == (seq.size + 1) // 2
        back = oracle.unpack_indices(12, seq.size, lo=lo, hi=hi)
        assert np.array_equal(back, seq)


def test_12bit_brute_force_bits():
    """Each index bit is read from the byte/nibble the reading assigns it to:
    set exactly one bit of one plane and check exactly one index changes."""
    n = 6
    for f in range(n):
        for bit in range(12):
            lo = np.zeros(n, dtype=np.uint8)
            hi = np.zeros((n + 1) // 2, dtype=np.uint8)
            if bit < 8:
                lo[f] = 1 << bit
            else:
                hi[f // 2] = 1 << ((bit - 8) + 4 * (f % 2))
            got = oracle.unpack_indices(12, n, lo=lo, hi=hi)
            want = np.zeros(n, dtype=np.int64)
            want[f] = 1 << bit
            assert np.array_equal(got, want), (f, bit)


def test_odd_count_pad_nibble_zero():
    lo, hi = oracle.pack_indices([0xFFF, 0xFFF, 0xFFF], 12)
    assert hi.tolist() == [0xFF, 0x0F]


def test_8bit_and_16bit():
    rng = np.random.default_rng(5)
    v8 = rng.integers(0, 256, 1000)
    lo, hi = oracle.pack_indices(v8, 8)
    assert hi is None and np.array_equal(oracle.unpack_indices(8, 1000, lo=lo), v8)
    v16 = rng.integers(0, 65536, 1000)
    p16, _ = oracle.pack_indices(v16, 16)
    assert p16.dtype == np.uint16
    assert np.array_equal(oracle.unpack_indices(16, 1000, idx16=p16), v16)
    # little-endian byte order of the stored uint16
    raw = np.array([0x34, 0x12, 0xFF, 0x00], dtype=np.uint8).view("<u2")
    assert oracle.unpack_indices(16, 2, idx16=raw).tolist() == [0x1234, 0x00FF]


def test_rejects_bad_width_and_range():
    with pytest.raises(ValueError):
        oracle.unpack_indices(10, 4, lo=np.zeros(4, np.uint8))
    with pytest.raises(ValueError):
        oracle.pack_indices([4096], 12)
    with pytest.raises(ValueError):
        oracle.pack_indices([-1], 8)


def test_exhaustive_4bit_roundtrip():
    """Every 4-bit value survives pack -> unpack at both nibble positions."""
    vals = np.arange(16)
    for seq in (np.repeat(vals, 2), np.tile(vals, 3), vals[:15], vals[::-1]):
        lo, hi = oracle.pack_indices(seq, 4)
        assert lo is None and hi.size == (seq.size + 1) // 2
        assert np.array_equal(oracle.unpack_indices(4, seq.size, hi=hi), seq)


def test_12bit_is_8bit_plane_plus_4bit_plane():
    """Structure of the bit-planes: a 12-bit index is the 8-bit index of its
    low plane plus 256 times the 4-bit index of its nibble plane."""
    rng = np.random.default_rng(17)
    n = 999
    lo = rng.integers(0, 256, n, dtype=np.uint8)
    hi = rng.integers(0, 256, (n + 1) // 2, dtype=np.uint8)
    i12 = oracle.unpack_indices(12, n, lo=lo, hi=hi)
    assert np.array_equal(i12, oracle.unpack_indices(8, n, lo=lo) + 256 * oracle.unpack_indices(4, n, hi=hi))


def test_4bit_brute_force_bits():
    n = 5
    for f in range(n):
        for bit in range(4):
            hi = np.zeros((n + 1) // 2, dtype=np.uint8)
            hi[f // 2] = 1 << (bit + 4 * (f % 2))
            want = np.zeros(n, dtype=np.int64)
            want[f] = 1 << bit
            assert np.array_equal(oracle.unpack_indices(4, n, hi=hi), want), (f, bit)
