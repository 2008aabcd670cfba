"""vq_gemm_noalloc (the many-token product on the library's static scratch)
against vq_gemm with a caller workspace, through the C ABI: the two share
their kernels, so outputs must be bit-identical, and both must meet the
oracle's bound.  Two calls in a row on one GPU, the second with fewer tokens
and a shorter K, show that what the first call leaves in the scratch does
not leak into the second; a call on the bf16 path (no scratch), a call with
a sparse correction and the over-limit error are covered too."""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import assert_within, device_weight, ensure_built, oracle_w64, x_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


def both(vq, w, xs, m, n):
    import torch
    x = x_to_device(xs, "bf16")
    ref = vq.vq_gemm(w, x)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    out = vq.vq_gemm_noalloc(w, x, y)
    torch.cuda.synchronize()
    assert out.data_ptr() == y.data_ptr()
    return ref.cpu().numpy(), y.cpu().numpy()


# (n, k, m, widths, seed) per call, in order: the second call is smaller
CALLS = [
    [(8320, 1024, 1900, [12, 12], 1), (1000, 512, 300, [12, 12], 2)],
    [(8448, 2048, 2000, [8, 8], 3), (8192, 256, 100, [12], 4), (4096, 512, 40, [12, 12], 5)],
]


@pytest.mark.parametrize("calls", CALLS, ids=["two", "three"])
def test_noalloc_matches_vq_gemm(vq, calls):
    for n, k, m, widths, seed in calls:
        print(f"noalloc {n}x{k} m={m} widths={widths}", flush=True)
        sw = vqsynth.random_weight(n, k, len(widths), widths, 128, seed=seed)
        xs, x64 = vqsynth.make_x(m, k, "bf16", np.random.SeedSequence(seed + 100))
        w = device_weight(sw)
        if m > 64:
            assert vq.vq_gemm_workspace_size(w, m) > 0, "this call should use the scratch"
        ref, got = both(vq, w, xs, m, n)
        np.testing.assert_array_equal(got, ref)
        y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
        assert_within(got, y_ref, bound, f"noalloc {n}x{k} m={m}")


def test_noalloc_sparse_correction(vq):
    n, k, m = 8448, 1024, 500
    sw = vqsynth.random_weight(n, k, 2, 12, 128, seed=11, sparse_density=0.002)
    xs, x64 = vqsynth.make_x(m, k, "bf16", np.random.SeedSequence(12))
    ref, got = both(vq, device_weight(sw), xs, m, n)
    np.testing.assert_array_equal(got, ref)
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(got, y_ref, bound, "noalloc sparse")


def test_noalloc_over_limit(vq):
    """More scratch than the static buffer holds: VQ_ERR_WORKSPACE, y untouched."""
    import torch
    sw = vqsynth.random_weight(1024, 8192, 2, 12, 128, seed=13)
    w = device_weight(sw)
    m = 2100  # 2100 x 8192 fp16 > 33 MiB
    assert vq.vq_gemm_workspace_size(w, m) > 33 << 20
    x = torch.zeros((m, 8192), dtype=torch.bfloat16, device="cuda")
    y = torch.full((m, 1024), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(vq.VQError) as e:
        vq.vq_gemm_noalloc(w, x, y)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
