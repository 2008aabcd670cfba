"""Parity of the 16-bit-index decode kernel with deep L2-gather pipelining
(one stage of 16-bit indices into a 65,536-entry codebook, GLQ page "How it
works" / "Bit widths") with the CPU oracle, through the C ABI.  Shapes route
to it: K % 2048 == 0, K <= 32768, scale blocks of whole 32-column units.  The
bar: |y - y_ref| <= 2e-3 sum|w x| + 1e-6.
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
