"""Pins for the storage-cost arithmetic.  orka README ("What this actually
is"): roughly 2 bits per weight, 8x smaller than fp16; 12 bits per group of 8
weights is 1.5 bits per weight per stage; GLQ "Bit widths": a 16-bit primary
index is 2 bpw."""
import pytest

import oracle

# (n_out, k_in, stages, bits, scale_block) -> total bytes incl. codebooks,
# worked by hand: stages*(index bytes) + 2*n_out*ceil(K/B_s) + stages*2^b*16
CASES = [
    ((256, 512, 1, 8, 512), 256 * 64 + 2 * 256 + 256 * 16),                      # 20,992
    ((576, 576, 1, 12, 128), 576 * 72 * 3 // 2 + 2 * 576 * 5 + 4096 * 16),       # 133,504
    ((1536, 576, 1, 12, 128), 1536 * 72 * 3 // 2 + 2 * 1536 * 5 + 4096 * 16),    # 246,784
    ((576, 1536, 1, 12, 128), 576 * 192 * 3 // 2 + 2 * 576 * 12 + 4096 * 16),   # 245,248
    ((4096, 4096, 2, 12, 128), 2 * 4096 * 512 * 3 // 2 + 2 * 4096 * 32 + 2 * 4096 * 16),
    ((14336, 4096, 2, 12, 128), 2 * 14336 * 512 * 3 // 2 + 2 * 14336 * 32 + 2 * 4096 * 16),
    ((4096, 14336, 2, 12, 128), 2 * 4096 * 1792 * 3 // 2 + 2 * 4096 * 112 + 2 * 4096 * 16),
    ((28672, 8192, 1, 16, 8192), 2 * 28672 * 1024 + 2 * 28672 + 65536 * 16),
    ((8192, 28672, 1, 16, 28672), 2 * 8192 * 3584 + 2 * 8192 + 65536 * 16),
]


@pytest.mark.parametrize("args,want", CASES)
def test_compressed_bytes(args, want):
    assert oracle.compressed_bytes(*args) == want


def test_known_totals():
    assert oracle.compressed_bytes(256, 512, 1, 8, 512) == 20992
    assert oracle.compressed_bytes(576, 576, 1, 12, 128) == 133504
    assert oracle.compressed_bytes(4096, 4096, 2, 12, 128) == 6684672
    assert oracle.compressed_bytes(14336, 4096, 2, 12, 128) == 23068672
    assert oracle.compressed_bytes(28672, 8192, 1, 16, 8192) == 59826176


def test_bits_per_weight():
    # 12 bits per 8 weights = 1.5 bpw per stage, plus 16 bits per scale block
    assert oracle.bits_per_weight(4096, 4096, 1, 12, 4096) == 1.5 + 16 / 4096
    assert oracle.bits_per_weight(4096, 4096, 2, 12, 128) == 3.125
    assert oracle.bits_per_weight(256, 512, 1, 8, 512) == 1.03125
    # a 16-bit primary index is 2 bpw (GLQ "Bit widths" table, 2 bpw row)
    assert oracle.bits_per_weight(28672, 8192, 1, 16, 8192) == 2 + 16 / 8192
    # orka: ~2 bits per weight is 8x smaller than fp16 (16 / 2)
    assert 16 / 2.0 == 8.0


def test_odd_group_count_pads_a_nibble():
    # 3 groups of 12-bit: 3 lo bytes + 2 hi bytes
    assert oracle.compressed_bytes(1, 24, 1, 12, 24, include_codebooks=False) == 3 + 2 + 2


def test_rvq_12_4_is_two_bits_per_weight():
    """orka README quick start: the rvq-12-4 mode gives about 2 bits per
    weight -- 12 + 4 index bits per group of 8 weights, plus the scales."""
    assert oracle.bits_per_weight(576, 576, 2, [12, 4], 576) == 2.0 + 16 / 576
    assert oracle.bits_per_weight(4096, 4096, 2, [12, 4], 128) == 2.125
    # stage bytes by hand: 12-bit = 1.5 B/group, 4-bit = 0.5 B/group
    g = 576 * 72
    assert oracle.compressed_bytes(576, 576, 2, [12, 4], 128, include_codebooks=False) == g * 3 // 2 + g // 2 + 2 * 576 * 5
    assert oracle.compressed_bytes(576, 576, 2, [12, 4], 128) == g * 2 + 2 * 576 * 5 + 4096 * 16 + 16 * 16


@pytest.mark.parametrize("widths,bpw", [([16], 2), ([16, 8], 3), ([16, 16], 4), ([16, 16, 8], 5),
                                        ([16, 16, 16], 6), ([16, 16, 16, 8], 7), ([16, 16, 16, 16], 8)])
def test_glq_bit_width_ladder(widths, bpw):
    """GLQ "Bit widths" table: a 16-bit primary, then 16- or 8-bit residual
    stages, gives 2..8 bits per weight (indices only; one scale per row adds
    16/K)."""
    k = 8192
    assert oracle.bits_per_weight(1024, k, len(widths), widths, k) == bpw + 16 / k


def test_4bit_odd_groups_and_codebook():
    # 3 groups of 4-bit: 2 bytes (pad nibble), one 16-entry fp16 codebook of 8-vectors = 256 B
    assert oracle.compressed_bytes(1, 24, 1, 4, 24, include_codebooks=False) == 2 + 2
    assert oracle.compressed_bytes(1, 24, 1, 4, 24) == 2 + 2 + 256
    with pytest.raises(ValueError):
        oracle.compressed_bytes(1, 24, 2, [12], 24)
    with pytest.raises(ValueError):
        oracle.compressed_bytes(1, 24, 1, [10], 24)
