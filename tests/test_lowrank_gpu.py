"""The low-rank correction (orka README, CLI: the correct command adds a
low-rank or sparse correction; the form W += U V is this library's reading)
through every entry point, against the oracle: the fp16 dequant bit for
bit, the products on every output within |y - y_ref| <= 2e-3 (sum|w x| +
sum_j |U| sum_k |V x|) + 1e-6."""
import numpy as np
import pytest

import vqsynth
from vqtest import (assert_all_rows, device_weight, ensure_built, oracle_indices, oracle_w16, x_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


# (n, k, stages, bits, scale_block, rank, sparse density): ranks that fill
# a wave's rows unevenly, rows not a multiple of any tile, k not a multiple
# of the 512-column chunk, the largest rank, a sparse correction beside it
SHAPES = [
    (1000, 1032, 2, 12, 128, 7, 0.0),
    (4096, 4096, 2, 12, 128, 32, 0.0),
    (640, 2048, 1, 8, 2048, 1, 0.0),
    (300, 520, 2, [12, 4], 40, 256, 0.0),
    (2048, 1024, 2, 12, 128, 16, 0.01),
    (8192, 4096, 1, 16, 4096, 24, 0.0),
]
IDS = [f"{n}x{k}-r{r}{'-sp' if sp else ''}" for n, k, _, _, _, r, sp in SHAPES]


def weight(shape, seed):
    n, k, st, bits, bs, r, sp = shape
    return vqsynth.random_weight(n, k, st, bits, bs, seed=seed, sparse_density=sp, lowrank_rank=r)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_dequant_bitexact(vq, shape):
    import torch
    print(f"lowrank dequant {shape}", flush=True)
    sw = weight(shape, 1)
    _, w_d = vq.vq_unpack_dequant(device_weight(sw), want_idx=False)
    torch.cuda.synchronize()
    want = oracle_w16(sw, None, oracle_indices(sw))
    assert np.array_equal(w_d.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("batch,dtype", [(1, "f32"), (1, "bf16"), (3, "bf16"), (16, "bf16"), (5, "f32")])
def test_gemv(vq, shape, batch, dtype):
    import torch
    print(f"lowrank gemv {shape} B={batch} {dtype}", flush=True)
    sw = weight(shape, 2)
    xs, x64 = vqsynth.make_x(batch, sw.k_in, dtype, np.random.SeedSequence(batch))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, dtype))
    torch.cuda.synchronize()
    assert_all_rows(y.cpu().numpy(), sw, x64, f"gemv {shape} B={batch}")


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
@pytest.mark.parametrize("m", [40, 300])
def test_gemm_and_noalloc(vq, shape, m):
    """vq_gemm with its workspace (the bf16 path at 40 tokens, the fp16 path
    at 300 where the format has one) and vq_gemm_noalloc, bit for bit the
    same."""
    import torch
    print(f"lowrank gemm {shape} m={m}", flush=True)
    sw = weight(shape, 3)
    w = device_weight(sw)
    xs, x64 = vqsynth.make_x(m, sw.k_in, "bf16", np.random.SeedSequence(m))
    x = x_to_device(xs, "bf16")
    need = vq.vq_gemm_workspace_size(w, m)
    assert need >= m * shape[5] * 4
    y = vq.vq_gemm(w, x, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    y2 = torch.empty_like(y)
    vq.vq_gemm_noalloc(w, x, y2)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.array_equal(got, y2.cpu().numpy())
    assert_all_rows(got, sw, x64, f"gemm {shape} m={m}")


@pytest.mark.parametrize("batch", [1, 16])
def test_llama8b_lowrank(vq, batch):
    """The Llama-3-8B linears with a rank-32 correction, every output."""
    import torch
    ws, act_ss = vqsynth.workload_weights("llama8b_lowrank")
    kids = act_ss.spawn(len(ws))
    for i, sw in enumerate(ws):
        print(f"llama8b_lowrank {sw.name} B={batch}", flush=True)
        xs, x64 = vqsynth.make_x(batch, sw.k_in, "bf16", kids[i])
        y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
        torch.cuda.synchronize()
        assert_all_rows(y.cpu().numpy(), sw, x64, f"llama8b_lowrank/{sw.name} B={batch}")


def test_gemv_rht_unsupported(vq):
    import torch
    sw = weight(SHAPES[-1], 4)
    w = device_weight(sw)
    x = torch.zeros((1, sw.k_in), dtype=torch.bfloat16, device="cuda")
    signs = torch.ones(sw.k_in, dtype=torch.int8, device="cuda")
    with pytest.raises(vq.VQError) as e:
        vq.vq_gemv_rht(w, x, signs, 4096)
    assert e.value.status == -4
