"""Parity of the fp16 matrix-core path of vq_gemm (more than 64 tokens, the
256-token tile kernels) with the CPU oracle, through the C ABI with the
caller's workspace.  x is converted once per call to fp16 with a
power-of-two rescale per token (exact), each weight is decoded to fp16 with
relative error at most 2^-10 + 2^-22 (two stages: sum, then scale, each
rounded once), and fp16 x fp16 products accumulate in fp32, so every output
meets |y - y_ref| <= 2e-3 sum|w x| + 1e-6 for any x with K <= 16384 (the
matmul acceptance bound), one-hot tokens included.  Every output is compared,
which covers every accumulator block of every tile, ragged ones included."""
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


def full_check(vq, sw, m, seed, what):
    import torch
    xs, x64 = vqsynth.make_x(m, sw.k_in, "bf16", np.random.SeedSequence(seed))
    w = device_weight(sw)
    need = vq.vq_gemm_workspace_size(w, m)
    assert need > 0, "this shape should take the fp16 tile path"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = vq.vq_gemm(w, x_to_device(xs, "bf16"), workspace=ws)
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    return assert_within(y.cpu().numpy(), y_ref, bound, what)


# (N, K, M, widths, seed): the wide kernel (256 x 256 tiles once there is one
# per CU) with ragged last tiles in both directions; the 256 x 128 tile
# kernel; one stage, 12+12, 12+4 and 8+8
@pytest.mark.parametrize("n,k,m,bits,seed", [
    (8320, 1024, 1900, 12, 1),          # wide, 12+12 (two stages below)
    (1000, 2048, 1900, 12, 2),          # tile kernel
    (8192, 512, 300, 8, 3),             # few token tiles: the tile kernel
    (16384, 256, 1024, 12, 4),          # wide, K = one trip of 8 steps
])
def test_gemm_f16_full(vq, n, k, m, bits, seed):
    print(f"f16 gemm {n}x{k} m={m}", flush=True)
    sw = vqsynth.random_weight(n, k, 2, bits, 128, seed=seed)
    worst = full_check(vq, sw, m, seed + 10, f"{n}x{k} m={m}")
    assert worst < 0.5, worst  # far inside the bound for dense x


@pytest.mark.parametrize("widths,rs", [([12], None), ([12, 4], None), ([8, 8], (0.2, 0.4)), ([12, 12], (0.5, 1.5))])
def test_gemm_f16_formats(vq, widths, rs):
    sw = vqsynth.random_weight(8448, 512, len(widths), widths, 128, seed=sum(widths), cb_sd=(0.02,) * len(widths),
                               stage_scale_range=rs)
    full_check(vq, sw, 2000, 7, f"{widths} rs={rs}")


def test_gemm_f16_one_hot(vq):
    """One-hot tokens recover decoded columns within the fp16 weight error
    (2^-10 + 2^-22 relative) and therefore within 2e-3 of |w| -- the bound
    the bf16 path cannot promise."""
    import torch
    n, k, m = 8448, 1024, 256
    sw = vqsynth.random_weight(n, k, 2, 12, 128, seed=77)
    cols = np.random.default_rng(78).choice(k, size=m, replace=True)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), cols] = 1.0
    xs = (x.view(np.uint32) >> 16).astype(np.uint16)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    w64 = oracle_w64(sw)
    got = y.cpu().numpy().astype(np.float64)
    want = w64[:, cols].T
    rel = np.abs(got - want) / np.maximum(np.abs(want), 2.0 ** -14)
    assert rel.max() <= 2.0 ** -10 + 2.0 ** -22 + 1e-9, rel.max()
    y_ref, bound = oracle.matmul_ref(w64, x.astype(np.float64))
    assert_within(got, y_ref, bound, "one-hot")


def test_gemm_f16_wide_range_tokens(vq):
    """Tokens whose values span 2^-20 .. 2^12 (and one all-zero token): the
    per-token power-of-two rescale keeps x exact in fp16."""
    import torch
    n, k, m = 8448, 512, 200
    sw = vqsynth.random_weight(n, k, 2, 12, 128, seed=88)
    rng = np.random.default_rng(89)
    x = (rng.standard_normal((m, k)) * np.exp2(rng.integers(-20, 13, (m, k)))).astype(np.float32)
    x[5] = 0.0
    xs = (x.view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation: exact values below
    x64 = (xs.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, "wide range")
    assert not y.cpu().numpy()[5].any()


def test_gemm_workspace_required(vq):
    """A call that needs a workspace and gets too little fails with
    VQ_ERR_WORKSPACE and launches nothing."""
    import torch
    sw = vqsynth.random_weight(8448, 512, 2, 12, 128, seed=5)
    w = device_weight(sw)
    need = vq.vq_gemm_workspace_size(w, 300)
    assert need >= 300 * 512 * 2
    x = torch.zeros((300, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vq.VQError) as e:
        vq.vq_gemm(w, x, workspace=torch.empty(need - 256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -8


@pytest.mark.parametrize("m", [63, 64, 65, 80])
def test_gemm_token_count_boundary(vq, m):
    """Either side of the switch from the few-token unit kernel (bf16 hi + lo
    weights, no workspace) to the fp16 tile path (more than 64 tokens, a
    workspace): the same 12+12 weight and one-hot, wide-range, sparse and
    dense tokens meet the 2e-3 bound on every output on both sides."""
    import torch
    from test_edges_gpu import _mixed_tokens
    sw = vqsynth.random_weight(2048, 1024, 2, 12, 128, seed=64)
    w = device_weight(sw)
    need = vq.vq_gemm_workspace_size(w, m)
    assert (need > 0) == (m > 64), need
    xs, x64 = _mixed_tokens(m, sw.k_in, m)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    y = vq.vq_gemm(w, x_to_device(xs, "bf16"), workspace=ws if need else None)
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"2048x1024 m={m}")
