"""Every entry point captured in a HIP graph and replayed: each replay must
write exactly what the eager call writes (the kernels are deterministic, so
bit for bit).  The output is poisoned with NaN before each replay, and eager
work (another call, torch ops, a synchronisation) runs between replays.  The
shapes route to the main kernels: the LDS and L2 decode GEMVs (the latter
also with the input transform inside), the fused and
the multi-token sparse correction, the few-token, wide and tile GEMMs, the RHT
and the LDS dequant, the codebook-sliced 16-bit GEMV (with and without the
transform inside), the shard-batched transform in both directions, the
no-allocation GEMM and the low-rank correction."""
import numpy as np
import pytest

import vqsynth
from vqtest import device_weight, ensure_built, x_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


def replay_matches(call, out, other):
    """Eager result of call() into out, then three graph replays against it."""
    import torch
    call()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        out.fill_(float("nan"))
        other()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int32) if out.dtype == torch.float32 else out.view(torch.int16),
                           want.view(torch.int32) if want.dtype == torch.float32 else want.view(torch.int16))
        assert same, f"replay {i} differs from the eager call"
    del g


def _x(m, k, xdt, seed):
    xs, _ = vqsynth.make_x(m, k, xdt, np.random.SeedSequence(seed))
    return x_to_device(xs, xdt)


# (name, N, K, widths, tokens, x dtype, sparse density, entry point)
CASES = [
    ("gemv_lds_b1", 4096, 4096, [12, 12], 1, "bf16", 0.0, "gemv"),
    ("gemv_l2_b1", 2048, 8192, [16], 1, "f32", 0.0, "gemv"),
    ("gemv_few_b16", 4096, 1024, [12, 12], 16, "bf16", 0.0, "gemv"),
    ("gemv_sparse_fused_b1", 2048, 2048, [12, 12], 1, "bf16", 0.01, "gemv"),
    ("gemv_sparse_b3", 2048, 2048, [12, 12], 3, "bf16", 0.01, "gemv"),
    ("gemm_wide", 8192, 512, [12, 12], 2048, "bf16", 0.0, "gemm"),
    ("gemm_tile", 1024, 256, [12, 12], 300, "bf16", 0.0, "gemm"),
    ("gemm_few_sparse", 4096, 1024, [12, 12], 40, "bf16", 0.01, "gemm"),
]


@pytest.mark.parametrize("name,n,k,widths,m,xdt,dens,entry", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_products(vq, name, n, k, widths, m, xdt, dens, entry):
    import torch
    sw = vqsynth.random_weight(n, k, len(widths), list(widths), 128, seed=n + k + m,
                               cb_sd=tuple(0.02 * 0.3 ** t for t in range(len(widths))), sparse_density=dens)
    w = device_weight(sw)
    x = _x(m, k, xdt, m)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    f = vq.vq_gemv if entry == "gemv" else vq.vq_gemm
    x2 = _x(m, k, xdt, m + 1)
    y2 = torch.empty_like(y)

    def other():
        f(w, x2, y=y2)
        torch.randn(1000, device="cuda").sum()

    replay_matches(lambda: f(w, x, y=y), y, other)


def test_graph_replay_rht(vq):
    import torch
    x = _x(2, 8192 + 2048, "bf16", 5)
    signs = torch.from_numpy(vqsynth.make_signs(8192 + 2048, np.random.SeedSequence(6))).cuda()
    out = torch.empty((2, 8192 + 2048), dtype=torch.float32, device="cuda")
    replay_matches(lambda: vq.rht_apply(x, signs, 8192, out=out), out, lambda: torch.ones(10, device="cuda").cumsum(0))


def test_graph_replay_gemv_rht(vq):
    import torch
    sw = vqsynth.random_weight(2048, 8192, 2, [16, 8], None, seed=8, cb_sd=(0.02, 0.02), stage_scale_range=(0.2, 0.4))
    w = device_weight(sw)
    x = _x(1, 8192, "bf16", 9)
    signs = torch.from_numpy(vqsynth.make_signs(8192, np.random.SeedSequence(10))).cuda()
    y = torch.empty((1, 2048), dtype=torch.float32, device="cuda")
    x2 = _x(1, 8192, "bf16", 11)
    y2 = torch.empty_like(y)
    replay_matches(lambda: vq.vq_gemv_rht(w, x, signs, 8192, y=y), y,
                   lambda: vq.vq_gemv_rht(w, x2, signs, 8192, y=y2))


def test_graph_replay_dequant(vq):
    import torch
    sw = vqsynth.random_weight(1024, 1024, 2, [12, 12], 128, seed=7, sparse_density=0.01)
    w = device_weight(sw)
    wt = torch.empty((1024, 1024), dtype=torch.float16, device="cuda")
    idx = torch.empty((2, 1024, 128), dtype=torch.int16, device="cuda")
    L = vq.lib()

    def call():
        st = L.vq_unpack_dequant(w.ref(), idx.data_ptr(), wt.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0

    replay_matches(call, wt, lambda: torch.zeros(10, device="cuda").add_(1))


def test_graph_replay_gemv_cbs(vq):
    """The codebook-sliced 16-bit kernel (one stage, one scale per row), plain
    and with the input transform inside."""
    import torch
    sw = vqsynth.random_weight(8192, 4096, 1, 16, 4096, seed=12)
    w = device_weight(sw)
    x = _x(1, 4096, "bf16", 13)
    x2 = _x(1, 4096, "bf16", 14)
    signs = torch.from_numpy(vqsynth.make_signs(4096, np.random.SeedSequence(15))).cuda()
    y = torch.empty((1, 8192), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    replay_matches(lambda: vq.vq_gemv(w, x, y=y), y, lambda: vq.vq_gemv(w, x2, y=y2))
    replay_matches(lambda: vq.vq_gemv_rht(w, x, signs, 4096, y=y), y, lambda: vq.vq_gemv(w, x2, y=y2))


def test_graph_replay_rht_shards(vq):
    import torch
    n = 8192 + 2048 + 576
    x = _x(3, n, "f32", 16)
    signs = torch.from_numpy(vqsynth.make_signs(n, np.random.SeedSequence(17))).cuda()
    out = torch.empty((3, n), dtype=torch.float32, device="cuda")
    for inverse in (False, True):
        replay_matches(lambda: vq.rht_apply_shards(x, signs, 4096, [8192, 2048, 576], inverse=inverse, out=out), out,
                       lambda: torch.ones(10, device="cuda").cumsum(0))


def test_graph_replay_noalloc_and_lowrank(vq):
    """vq_gemm_noalloc (static scratch) and a weight with a low-rank
    correction through vq_gemv (one launch more) and vq_gemm (t in the
    workspace)."""
    import torch
    sw = vqsynth.random_weight(4096, 1024, 2, [12, 12], 128, seed=18, lowrank_rank=16)
    w = device_weight(sw)
    for m, f in ((300, lambda x, y: vq.vq_gemm_noalloc(w, x, y)), (300, lambda x, y: vq.vq_gemm(w, x, y=y)),
                 (1, lambda x, y: vq.vq_gemv(w, x, y=y)), (16, lambda x, y: vq.vq_gemv(w, x, y=y))):
        x = _x(m, 1024, "bf16", 19 + m)
        x2 = _x(m, 1024, "bf16", 20 + m)
        y = torch.empty((m, 4096), dtype=torch.float32, device="cuda")
        y2 = torch.empty_like(y)
        replay_matches(lambda: f(x, y), y, lambda: f(x2, y2))
