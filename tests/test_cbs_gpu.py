"""Parity of the codebook-sliced decode kernel (one stage of 16-bit indices
into a 65,536-entry codebook, GLQ page "How it works" / "Bit widths"; the
codebook streamed through LDS in slices) with the CPU oracle, through the C
ABI.  Weights of at least 2^25 entries with one scale per row and
K = 1024 U x {1, 2, 4, 8} route to it.  The bar: |y - y_ref| <= 2e-3 sum|w x|
+ 1e-6 per output.  Large outputs are compared on sampled rows plus the
first and last rows of every workgroup's block (where the row split and the
K-part sums meet)."""
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


def block_edges(n, cus=256):
    """First and last row of every workgroup's block of the persistent grid
    (a superset of the launch's real split for any grid up to `cus`)."""
    per = -(-n // cus)
    rows = set()
    for b in range(0, n, per):
        rows |= {b, min(n, b + per) - 1}
    return rows


def check_rows(sw, y, x64, rows, what):
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), x64)
    return assert_within(y[:, rows], y_ref, bound, what)


# (N, K, x dtype, seed): pairs per lane U = 4 (K 8192, 16384, 32768), 7
# (K 28672), 2 (K 2048) and 1 (K 1024); fewer rows per wave than it holds,
# ragged row counts, and two row chunks per workgroup (40000 x 8192)
CASES = [(4096, 8192, "bf16", 1), (28672, 8192, "bf16", 2), (8192, 28672, "f32", 3), (4100, 16384, "bf16", 4),
         (1024, 32768, "f32", 5), (65536, 1024, "bf16", 6), (33000, 2048, "f32", 7), (40000, 8192, "bf16", 8)]


@pytest.mark.parametrize("n,k,xdt,seed", CASES)
def test_cbs_gemv(vq, n, k, xdt, seed):
    import torch
    print(f"cbs {n}x{k} {xdt}", flush=True)
    sw = vqsynth.random_weight(n, k, 1, 16, None, seed=100 + seed)
    xs, x64 = vqsynth.make_x(1, k, xdt, np.random.SeedSequence(200 + seed))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_rows(n, 64, seed).tolist()) | block_edges(n)))
    check_rows(sw, y.cpu().numpy(), x64, rows, f"{n}x{k} {xdt}")


def test_cbs_gemv_stage_scale(vq):
    """A single 16-bit stage with a residual scale: w = s r0 cb[idx]."""
    import torch
    sw = vqsynth.random_weight(8192, 8192, 1, 16, None, seed=11, stage_scale_range=(0.2, 0.4))
    sw.stage_scales = np.array([0.3], np.float32)  # the generator keeps the primary's at 1
    xs, x64 = vqsynth.make_x(1, 8192, "bf16", np.random.SeedSequence(12))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    check_rows(sw, y.cpu().numpy(), x64, sample_rows(8192, 128, 13), "stage scale")


def test_cbs_gemv_one_hot(vq):
    """One-hot x recovers dequantized columns exactly: the codebook entry
    times 1 is exact, every other product and sum adds zeros, and the row
    scale multiplies once (the fp32 product of two fp16 values is exact)."""
    import torch
    n, k = 4096, 8192
    sw = vqsynth.random_weight(n, k, 1, 16, None, seed=21)
    w = device_weight(sw)
    rows = sample_rows(n, 256, 22)
    w64 = oracle_w64(sw, rows)
    for c in (0, 7, 4095, 4096, 8191):
        x = np.zeros((1, k), np.float32)
        x[0, c] = 1.0
        for xdt in ("f32", "bf16"):
            xs = x if xdt == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)
            y = vq.vq_gemv(w, x_to_device(xs, xdt))
            torch.cuda.synchronize()
            got = y.cpu().numpy()[0, rows].astype(np.float64)
            assert np.array_equal(got, w64[:, c]), (c, xdt, np.abs(got - w64[:, c]).max())


def test_cbs_gemv_zero_and_range(vq):
    """x = 0 gives exactly 0; x spanning 2^-20 .. 2^12 within every lane's
    columns stays inside the bound (the per-lane power-of-two rescale)."""
    import torch
    n, k = 4096, 8192
    sw = vqsynth.random_weight(n, k, 1, 16, None, seed=31)
    w = device_weight(sw)
    y = vq.vq_gemv(w, torch.zeros((1, k), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert not y.cpu().numpy().any()
    rng = np.random.default_rng(32)
    x = (rng.standard_normal(k) * np.exp2(rng.integers(-20, 13, k))).astype(np.float32)[None]
    y = vq.vq_gemv(w, x_to_device(x, "f32"))
    torch.cuda.synchronize()
    check_rows(sw, y.cpu().numpy(), x.astype(np.float64), sample_rows(n, 128, 33), "wide range")


def test_cbs_gemv_deterministic(vq):
    """Two launches give bit-identical outputs (fixed reduction order)."""
    import torch
    sw = vqsynth.random_weight(28672, 8192, 1, 16, None, seed=41)
    w = device_weight(sw)
    xs, _ = vqsynth.make_x(1, 8192, "bf16", np.random.SeedSequence(42))
    x = x_to_device(xs, "bf16")
    a = vq.vq_gemv(w, x).cpu().numpy()
    b = vq.vq_gemv(w, x).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# (N, K, x dtype, largest transform block): the input transform inside the
# sliced kernel (vq_gemv_rht): blocks of 8192 as in the 70B-MLP workload,
# greedy blocks of a non-power-of-two K (28672 -> 8192 x 3 + 4096), small
# blocks (16, below the 16-element register staging; 1: signs only)
RHT_CASES = [(28672, 8192, "bf16", 8192), (8192, 28672, "bf16", 8192), (4096, 16384, "f32", 16384),
             (8192, 8192, "bf16", 16), (4096, 8192, "f32", 1), (33000, 2048, "bf16", 512)]


@pytest.mark.parametrize("n,k,xdt,mb", RHT_CASES)
def test_cbs_gemv_rht(vq, n, k, xdt, mb):
    import torch
    print(f"cbs rht {n}x{k} {xdt} mb={mb}", flush=True)
    sw = vqsynth.random_weight(n, k, 1, 16, None, seed=n + k + mb)
    xs, x64 = vqsynth.make_x(2, k, xdt, np.random.SeedSequence(k + mb))
    signs = vqsynth.make_signs(k, np.random.SeedSequence(mb + 3))
    y = vq.vq_gemv_rht(device_weight(sw), x_to_device(xs, xdt), torch.from_numpy(signs).cuda(), mb)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_rows(n, 48, mb).tolist()) | block_edges(n)))
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), oracle.rht_ref(x64, signs, mb))
    assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"rht {n}x{k} {xdt} mb={mb}")


# A 16-bit primary plus an 8-bit residual stage (GLQ page, "Advanced > Bit
# widths": the 16 + 8 ladder) on the sliced kernel, the residual's codebook in
# LDS beside the slice and its pass after the slices: every pairs-per-lane
# instance (U = 4, 7, 4, 1, 2, 8), with and without stage scales, bf16 and
# fp32 x.
RES_CASES = [(4096, 8192, "bf16", (0.2, 0.4), 31), (8192, 28672, "f32", (0.2, 0.4), 32),
             (4100, 16384, "bf16", None, 33), (32768, 1024, "f32", (0.5, 1.5), 34),
             (16384, 2048, "bf16", None, 35), (512, 65536, "bf16", (0.2, 0.4), 36)]


@pytest.mark.parametrize("n,k,xdt,ss,seed", RES_CASES)
def test_cbs_gemv_residual(vq, n, k, xdt, ss, seed):
    import torch
    print(f"cbs 16+8 {n}x{k} {xdt} {ss}", flush=True)
    sw = vqsynth.random_weight(n, k, 2, [16, 8], None, seed=100 + seed, cb_sd=(0.02, 0.02), stage_scale_range=ss)
    xs, x64 = vqsynth.make_x(1, k, xdt, np.random.SeedSequence(200 + seed))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_rows(n, 64, seed).tolist()) | block_edges(n)))
    check_rows(sw, y.cpu().numpy(), x64, rows, f"16+8 {n}x{k} {xdt}")


def test_cbs_gemv_residual_every_output(vq):
    """Every output of a 16 + 8 weight with stage scales (4096 x 8192)."""
    import torch
    n, k = 4096, 8192
    sw = vqsynth.random_weight(n, k, 2, [16, 8], None, seed=141, cb_sd=(0.02, 0.02), stage_scale_range=(0.2, 0.4))
    xs, x64 = vqsynth.make_x(1, k, "bf16", np.random.SeedSequence(142))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    for r0 in range(0, n, 1024):
        check_rows(sw, got, x64, np.arange(r0, r0 + 1024), f"16+8 every output, rows {r0}..")


@pytest.mark.parametrize("n,k,seed", [(4096, 8192, 51), (8192, 28672, 52)])
def test_cbs_gemv_residual_rht_fused(vq, n, k, seed):
    """The input transform inside the kernel, then the 16 + 8 product."""
    import torch
    sw = vqsynth.random_weight(n, k, 2, [16, 8], None, seed=100 + seed, cb_sd=(0.02, 0.02),
                               stage_scale_range=(0.2, 0.4))
    xs, x64 = vqsynth.make_x(1, k, "bf16", np.random.SeedSequence(200 + seed))
    signs = vqsynth.make_signs(k, np.random.SeedSequence(300 + seed))
    y = vq.vq_gemv_rht(device_weight(sw), x_to_device(xs, "bf16"), torch.from_numpy(signs).cuda(), 8192)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_rows(n, 64, seed).tolist()) | block_edges(n)))
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), oracle.rht_ref(x64, signs, 8192))
    assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"16+8 fused transform {n}x{k}")


# Two 16-bit stages (GLQ page, "Advanced > Bit widths": the 16 + 16 ladder):
# the second stage's codebook streams through the slices after the first's,
# its indices loaded into the same registers at the switch.  A second stage
# scaled by 0 adds nothing and runs as one stage.
ST2_CASES = [(4096, 8192, "bf16", (0.2, 0.4), 61), (8192, 28672, "f32", None, 62),
             (32768, 1024, "bf16", (0.5, 1.5), 63), (512, 65536, "f32", (0.2, 0.4), 64)]


@pytest.mark.parametrize("n,k,xdt,ss,seed", ST2_CASES)
def test_cbs_gemv_two_16bit_stages(vq, n, k, xdt, ss, seed):
    import torch
    print(f"cbs 16+16 {n}x{k} {xdt} {ss}", flush=True)
    sw = vqsynth.random_weight(n, k, 2, [16, 16], None, seed=100 + seed, cb_sd=(0.02, 0.006), stage_scale_range=ss)
    xs, x64 = vqsynth.make_x(1, k, xdt, np.random.SeedSequence(200 + seed))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_rows(n, 64, seed).tolist()) | block_edges(n)))
    check_rows(sw, y.cpu().numpy(), x64, rows, f"16+16 {n}x{k} {xdt}")


def test_cbs_gemv_two_16bit_stages_every_output(vq):
    """Every output of a 16 + 16 weight with stage scales (4096 x 8192),
    and the same weight with the second stage scaled by 0."""
    import torch
    n, k = 4096, 8192
    sw = vqsynth.random_weight(n, k, 2, [16, 16], None, seed=171, cb_sd=(0.02, 0.02), stage_scale_range=(0.2, 0.4))
    xs, x64 = vqsynth.make_x(1, k, "bf16", np.random.SeedSequence(172))
    for r1 in (None, 0.0):
        if r1 is not None:
            sw.stage_scales = np.array([sw.stage_scales[0], r1], np.float32)
        y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        for r0 in range(0, n, 1024):
            check_rows(sw, got, x64, np.arange(r0, r0 + 1024), f"16+16 r1={r1} rows {r0}..")


def test_cbs_gemv_two_16bit_stages_rht_fused(vq):
    import torch
    n, k = 8192, 28672
    sw = vqsynth.random_weight(n, k, 2, [16, 16], None, seed=181, cb_sd=(0.02, 0.02), stage_scale_range=(0.2, 0.4))
    xs, x64 = vqsynth.make_x(1, k, "bf16", np.random.SeedSequence(182))
    signs = vqsynth.make_signs(k, np.random.SeedSequence(183))
    y = vq.vq_gemv_rht(device_weight(sw), x_to_device(xs, "bf16"), torch.from_numpy(signs).cuda(), 8192)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(sample_rows(n, 64, 184).tolist()) | block_edges(n)))
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), oracle.rht_ref(x64, signs, 8192))
    assert_within(y.cpu().numpy()[:, rows], y_ref, bound, "16+16 fused transform")
