"""The Python binding rejects mis-shaped, mis-typed and host tensors before
calling the library.  The C ABI cannot see buffer sizes, so these checks are
what stands between a wrong tensor and an out-of-bounds kernel access.  They
run without a GPU: every case raises before any HIP call."""
import numpy as np
import pytest
import torch

import compressed_index_matmul_amd as vq
import vqsynth


def cpu_weight(sw, **over):
    kw = dict(codebooks=sw.codebooks, scales=sw.scales, lo=sw.lo, hi=sw.hi, idx16=sw.idx16, device="cpu",
              stage_bits=sw.stage_bits, stage_scales=sw.stage_scales, sparse=sw.sparse)
    kw.update(over)
    return vq.VQWeight(sw.n_out, sw.k_in, sw.n_stages, sw.idx_bits, sw.scale_block, **kw)


@pytest.fixture(scope="module")
def sw12():
    return vqsynth.random_weight(16, 64, 2, 12, 32, seed=5)


def test_weight_arrays_accepted(sw12):
    w = cpu_weight(sw12)
    assert w.widths() == [12, 12]


@pytest.mark.parametrize("field,bad", [
    ("lo", lambda sw: [sw.lo[0][:-1], sw.lo[1]]),                 # low plane one byte short
    ("hi", lambda sw: [sw.hi[0], np.concatenate([sw.hi[1], [0]])]),  # nibble plane one byte long
    ("codebooks", lambda sw: [sw.codebooks[0][:-1], sw.codebooks[1]]),
    ("codebooks", lambda sw: [sw.codebooks[0]]),                  # a stage without its codebook
    ("scales", lambda sw: sw.scales[:-1]),
    ("lo", lambda sw: [sw.lo[0]]),                                # stage 1's low plane missing
])
def test_weight_array_lengths(sw12, field, bad):
    with pytest.raises(ValueError):
        cpu_weight(sw12, **{field: bad(sw12)})


def test_weight_16bit_and_sparse_lengths():
    sw = vqsynth.random_weight(8, 64, 1, 16, None, seed=3)
    cpu_weight(sw)
    with pytest.raises(ValueError):
        cpu_weight(sw, idx16=[sw.idx16[0][:-2]])
    sw = vqsynth.random_weight(8, 64, 1, 8, 32, seed=4, sparse_density=0.1)
    cpu_weight(sw)
    rp, cl, vl = sw.sparse
    with pytest.raises(ValueError):
        cpu_weight(sw, sparse=(rp[:-1], cl, vl))
    with pytest.raises(ValueError):
        cpu_weight(sw, sparse=(rp, cl, vl[:-1]))


def test_host_weight_rejected_by_compute_calls(sw12):
    w = cpu_weight(sw12)
    x = torch.zeros((1, sw12.k_in), dtype=torch.bfloat16)
    for call in (lambda: vq.vq_gemv(w, x), lambda: vq.vq_gemm(w, x), lambda: vq.vq_unpack_dequant(w)):
        with pytest.raises(ValueError, match="GPU"):
            call()


class _FakeGpuWeight:
    """Stand-in with a GPU device and no device memory: the argument checks
    run (and raise) before anything would dereference it."""

    def __init__(self, n=16, k=64):
        self.n_out, self.k_in, self.n_stages = n, k, 1
        self.device = torch.device("cuda:0")

    def ref(self):  # pragma: no cover - never reached
        raise AssertionError("the library was called")


@pytest.mark.parametrize("x,err", [
    (torch.zeros((1, 63), dtype=torch.bfloat16), ValueError),     # K mismatch
    (torch.zeros((2, 3, 64), dtype=torch.bfloat16), ValueError),  # not [tokens, K]
    (torch.zeros((1, 64), dtype=torch.float16), TypeError),       # dtype
    (torch.zeros((1, 64), dtype=torch.bfloat16), ValueError),     # host tensor
    (torch.zeros((64, 2), dtype=torch.float32).t(), ValueError),   # [2, 64] view, not contiguous... and K != 64
])
def test_gemv_x_checks(x, err):
    with pytest.raises(err):
        vq.vq_gemv(_FakeGpuWeight(), x)


def test_gemv_token_count_and_y_checks():
    w = _FakeGpuWeight()
    with pytest.raises(ValueError):
        vq.vq_gemv(w, torch.zeros((17, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        vq.vq_gemv_rht(w, torch.zeros((1, 64), dtype=torch.float32), torch.ones(64, dtype=torch.int8), 64)


def test_gemm_checks():
    w = _FakeGpuWeight()
    with pytest.raises(TypeError):
        vq.vq_gemm(w, torch.zeros((4, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        vq.vq_gemm(w, torch.zeros((4, 65), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        vq.vq_gemm(w, torch.zeros((4, 64), dtype=torch.bfloat16))  # host x


def test_rht_checks():
    x = torch.zeros((1, 64), dtype=torch.float32)
    with pytest.raises(ValueError):  # host tensors
        vq.rht_apply(x, torch.ones(64, dtype=torch.int8), 64)
    with pytest.raises(TypeError):
        vq.rht_apply(torch.zeros((1, 64), dtype=torch.float16), torch.ones(64, dtype=torch.int8), 64)
    with pytest.raises(ValueError):
        vq.rht_apply(torch.zeros((2, 2, 2)), torch.ones(8, dtype=torch.int8), 8)
