"""The product with the input transform inside the 16-bit decode kernel
(vq_gemv_rht; GLQ page, "Advanced", "Trellis codebook": the input Hadamard
transform runs in every decode block) against the oracle's exact transform
and exact product, through the C ABI.  Bar: |y - y_ref| <= 2e-3 sum|w x'| +
1e-6 with x' the exact transform (the fp32 transform's own error is far
below it)."""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import assert_all_rows, assert_within, device_weight, ensure_built, oracle_w64, sample_rows, x_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


def make(n, k, widths, rs, bs, seed):
    sd = (0.02, 0.02 if rs else 0.006)[: len(widths)]
    return vqsynth.random_weight(n, k, len(widths), list(widths), bs, seed=seed, cb_sd=sd, stage_scale_range=rs)


# (N, K, widths, stage-scale range, scale block, max_block, x dtype, tokens):
# one block shorter than max_block, one whole block, four blocks of two
# sizes, two blocks, small blocks, a residual stage with stage scales
CASES = [(300, 2048, (16,), None, None, 8192, "bf16", 1), (517, 8192, (16,), None, 128, 8192, "f32", 1),
         (260, 28672, (16,), None, None, 8192, "bf16", 2), (333, 6144, (16, 8), (0.2, 0.4), 128, 4096, "bf16", 1),
         (129, 4096, (16, 16), (0.3, 0.5), 32, 256, "f32", 3), (64, 2048, (16,), None, 64, 1, "bf16", 1),
         (1000, 8192, (16, 8), (0.2, 0.4), None, 16384, "bf16", 1)]


@pytest.mark.parametrize("n,k,widths,rs,bs,mb,xdt,m", CASES)
def test_gemv_rht(vq, n, k, widths, rs, bs, mb, xdt, m):
    import torch
    sw = make(n, k, widths, rs, bs, n + k)
    xs, x64 = vqsynth.make_x(m, k, xdt, np.random.SeedSequence(k + m))
    signs = vqsynth.make_signs(k, np.random.SeedSequence(k + 1))
    y = vq.vq_gemv_rht(device_weight(sw), x_to_device(xs, xdt), torch.from_numpy(signs).cuda(), mb)
    torch.cuda.synchronize()
    rows = None if n * k <= (1 << 22) else sample_rows(n, 96, 8)
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), oracle.rht_ref(x64, signs, mb))
    got = y.cpu().numpy() if rows is None else y.cpu().numpy()[:, rows]
    assert_within(got, y_ref, bound, f"{widths} rs={rs} {n}x{k} mb={mb} {xdt} B={m}")


def test_gemv_rht_matches_separate_launches(vq):
    """rht_apply then vq_gemv gives the same product to the same bar."""
    import torch
    sw = make(2048, 8192, (16,), None, None, 5)
    xs, x64 = vqsynth.make_x(1, 8192, "bf16", np.random.SeedSequence(6))
    signs = torch.from_numpy(vqsynth.make_signs(8192, np.random.SeedSequence(7))).cuda()
    w = device_weight(sw)
    x = x_to_device(xs, "bf16")
    fused = vq.vq_gemv_rht(w, x, signs, 8192)
    sep = vq.vq_gemv(w, vq.rht_apply(x, signs, 8192))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), oracle.rht_ref(x64, signs.cpu().numpy(), 8192))
    assert_within(fused.cpu().numpy(), y_ref, bound, "fused")
    assert_within(sep.cpu().numpy(), y_ref, bound, "separate")


def test_gemv_rht_unsupported(vq):
    """A 12-bit weight: VQ_ERR_UNSUPPORTED, the output untouched."""
    import torch
    from compressed_index_matmul_amd import VQError
    sw = make(64, 2048, (12,), None, None, 3)
    x = x_to_device(vqsynth.make_x(1, 2048, "bf16", np.random.SeedSequence(1))[0], "bf16")
    signs = torch.from_numpy(vqsynth.make_signs(2048, np.random.SeedSequence(2))).cuda()
    y = torch.full((1, 64), 7.0, device="cuda")
    with pytest.raises(VQError):
        vq.vq_gemv_rht(device_weight(sw), x, signs, 2048, y=y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


def test_gemv_rht_mlp70b(vq):
    """The 70B-MLP linears with the transform fused: every output against the
    oracle's exact transform and product."""
    import torch
    ws, act_ss = vqsynth.workload_weights("mlp70b")
    kids = act_ss.spawn(2 * len(ws))
    for i, sw in enumerate(ws):
        xs, x64 = vqsynth.make_x(1, sw.k_in, "bf16", kids[i])
        signs = vqsynth.make_signs(sw.k_in, kids[len(ws) + i])
        y = vq.vq_gemv_rht(device_weight(sw), x_to_device(xs, "bf16"), torch.from_numpy(signs).cuda(), 8192)
        torch.cuda.synchronize()
        assert_all_rows(y.cpu().numpy(), sw, oracle.rht_ref(x64, signs, 8192), f"mlp70b/{sw.name} fused")
