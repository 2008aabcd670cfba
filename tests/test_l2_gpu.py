"""Parity of the 16-bit-index decode kernel with deep L2-gather pipelining
(a stage of 16-bit indices into a 65,536-entry codebook, GLQ page "How it
works" / "Bit widths", alone or with an 8- or 16-bit residual stage and stage
scales) with the CPU oracle, through the C ABI.  Shapes route to it: K % 2048
== 0, K <= 32768 (less with a residual), scale blocks of 32-column units that
divide 2048 or cover the row.  The bar: |y - y_ref| <= 2e-3 sum|w x| + 1e-6.
"""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import assert_within, device_weight, ensure_built, oracle_w64, sample_rows, x_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


# (N, K, scale block (None = per row), x dtype): fewer rows than waves, uneven
# row blocks, 32-column and 128-column scale blocks, 1..14 units per lane
CASES = [(7, 2048, None, "f32"), (1000, 4096, None, "bf16"), (2057, 8192, 32, "f32"), (333, 6144, 128, "bf16"),
         (4099, 2048, None, "bf16"), (512, 28672, None, "f32"), (300, 32768, 2048, "bf16")]


@pytest.mark.parametrize("n,k,bs,xdt", CASES)
def test_l2_gemv(vq, n, k, bs, xdt):
    import torch
    sw = vqsynth.random_weight(n, k, 1, 16, bs, seed=n + k)
    xs, x64 = vqsynth.make_x(1, k, xdt, np.random.SeedSequence(k + 1))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    rows = None if n * k <= (1 << 22) else sample_rows(n, 96, 5)
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), x64)
    got = y.cpu().numpy() if rows is None else y.cpu().numpy()[:, rows]
    assert_within(got, y_ref, bound, f"{n}x{k} bs={bs} {xdt}")


def test_l2_gemv_one_hot(vq):
    """One-hot x recovers dequantized columns: the codebook entry times the
    scale, one fp32 rounding."""
    import torch
    sw = vqsynth.random_weight(1024, 4096, 1, 16, 128, seed=9)
    w = device_weight(sw)
    w64 = oracle_w64(sw)
    for c in (0, 31, 2049, 4095):
        x = np.zeros((1, 4096), np.float32)
        x[0, c] = 1.0
        y = vq.vq_gemv(w, torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        assert np.allclose(y.cpu().numpy()[0].astype(np.float64), w64[:, c], rtol=2 ** -22, atol=0), c


def test_l2_gemv_batch_tokens(vq):
    """fp32 tokens run one launch each; every token against the oracle."""
    import torch
    sw = vqsynth.random_weight(800, 4096, 1, 16, None, seed=3)
    xs, x64 = vqsynth.make_x(3, 4096, "f32", np.random.SeedSequence(4))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "f32"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, "800x4096 B=3")


# (widths, stage-scale range, N, K, scale block, x dtype): a 16-bit primary
# with an 8-bit or a 16-bit residual, with and without stage scales; K up to
# the most units per lane each residual width takes (14 for 8 bits, 13 for 16
# bits), and past it (the general kernel) for the 16-bit residual
LADDERS = [((16, 8), (0.2, 0.4), 1000, 8192, 128, "bf16"), ((16, 8), None, 333, 28672, None, "f32"),
           ((16, 16), (0.2, 0.4), 2057, 4096, 32, "f32"), ((16, 16), None, 517, 26624, 2048, "bf16"),
           ((16, 16), (0.3, 0.5), 260, 28672, None, "bf16"), ((16, 8), (0.25, 0.5), 7, 2048, None, "bf16")]


@pytest.mark.parametrize("widths,rs,n,k,bs,xdt", LADDERS)
def test_l2_gemv_ladder(vq, widths, rs, n, k, bs, xdt):
    import torch
    sd = (0.02, 0.02 if rs else 0.006)
    sw = vqsynth.random_weight(n, k, 2, list(widths), bs, seed=n + 3 * k, cb_sd=sd, stage_scale_range=rs)
    xs, x64 = vqsynth.make_x(1, k, xdt, np.random.SeedSequence(k + 7))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    rows = None if n * k <= (1 << 22) else sample_rows(n, 96, 6)
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), x64)
    got = y.cpu().numpy() if rows is None else y.cpu().numpy()[:, rows]
    assert_within(got, y_ref, bound, f"{widths} rs={rs} {n}x{k} bs={bs} {xdt}")


def test_l2_gemv_block_not_dividing_2048(vq):
    """A scale block of 96 columns takes the general kernel; same bar."""
    import torch
    sw = vqsynth.random_weight(300, 6144, 1, 16, 96, seed=12)
    xs, x64 = vqsynth.make_x(1, 6144, "bf16", np.random.SeedSequence(13))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, "300x6144 bs=96")


def test_l2_gemv_ladder_sparse(vq):
    """16+8 with stage scales and a sparse correction (added by its own
    kernel after the product)."""
    import torch
    sw = vqsynth.random_weight(700, 4096, 2, [16, 8], 128, seed=21, cb_sd=(0.02, 0.02), stage_scale_range=(0.2, 0.4),
                               sparse_density=0.01)
    xs, x64 = vqsynth.make_x(1, 4096, "bf16", np.random.SeedSequence(22))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, "16+8/rs sparse")
