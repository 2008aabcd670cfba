"""The largest weights the descriptor allows (n_out * k_in just below 2^31)
on each kernel family, so that every 32-bit offset in the kernels is
exercised near its limit: two 12-bit stages on the LDS decode kernel, the
fp16 wide GEMM and the dequant; 16-bit indices on the L2-gather and the
codebook-sliced decode kernels.  Outputs are checked on sampled rows (the
first, the last and random ones) that the oracle unpacks and decodes one by
one; indices and the fp16 dequant bit for bit, products within the bound."""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import assert_within, device_weight, ensure_built, oracle_w64, x_to_device

pytestmark = pytest.mark.gpu

LIMIT = 1 << 31


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


def rows_of(n, seed, count=48):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set(rng.choice(n, count, replace=False).tolist()) | {0, 1, n - 2, n - 1}))


def row_indices(sw, rows):
    """Per stage, the unpacked indices of the given rows only (the planes are
    sliced per row; every row here holds an even number of groups)."""
    g = sw.k_in // 8
    assert g % 2 == 0
    out = []
    for t, b in enumerate(sw.widths):
        parts = []
        for r in rows:
            lo = sw.lo[t][r * g:(r + 1) * g] if sw.lo[t] is not None else None
            hi = sw.hi[t][r * g // 2:(r + 1) * g // 2] if sw.hi[t] is not None else None
            i16 = sw.idx16[t][r * g:(r + 1) * g] if sw.idx16[t] is not None else None
            parts.append(oracle.unpack_indices(b, g, lo=lo, hi=hi, idx16=i16))
        out.append(np.concatenate(parts))
    return out


def rows_w64(sw, rows, idx):
    return oracle.dequant_exact(len(rows), sw.k_in, idx, sw.codebooks, sw.scales[rows], sw.scale_block,
                                sw.stage_scales)


def test_max_12bit_two_stages(vq):
    import torch
    n, k = LIMIT // 4096 - 1, 4096
    assert n * k < LIMIT
    print(f"max 12+12: {n} x {k}", flush=True)
    sw = vqsynth.random_weight(n, k, 2, 12, 128, seed=1)
    w = device_weight(sw)
    rows = rows_of(n, 2)
    idx = row_indices(sw, rows)
    w64 = rows_w64(sw, rows, idx)
    # decode kernel, one bf16 token
    xs, x64 = vqsynth.make_x(1, k, "bf16", np.random.SeedSequence(3))
    y = vq.vq_gemv(w, x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(w64, x64)
    assert_within(y.cpu().numpy()[:, rows], y_ref, bound, "max 12+12 gemv")
    del y
    # fp16 wide GEMM, 100 tokens
    xs, x64 = vqsynth.make_x(100, k, "bf16", np.random.SeedSequence(4))
    y = vq.vq_gemm(w, x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(w64, x64)
    assert_within(y[:, torch.from_numpy(rows).cuda()].cpu().numpy(), y_ref, bound, "max 12+12 gemm")
    del y
    # dequant: indices and fp16 weights of the sampled rows
    idx_d, w_d = vq.vq_unpack_dequant(w)
    torch.cuda.synchronize()
    r = torch.from_numpy(rows).cuda()
    got_idx = idx_d[:, r].cpu().numpy().view(np.uint16).reshape(2, -1)
    for t in range(2):
        assert np.array_equal(got_idx[t].astype(np.int64), idx[t]), f"stage {t} indices"
    want = oracle.dequant_fp16(len(rows), k, idx, sw.codebooks, sw.scales[rows], sw.scale_block)
    assert np.array_equal(w_d[r].cpu().numpy().view(np.uint16), want.view(np.uint16)), "fp16 weights"


@pytest.mark.parametrize("n,k,kernel", [(69904, 30720, "L2 gather"), (74897, 28672, "codebook slices")])
def test_max_16bit(vq, n, k, kernel):
    import torch
    assert n * k < LIMIT
    print(f"max 16-bit ({kernel}): {n} x {k}", flush=True)
    sw = vqsynth.random_weight(n, k, 1, 16, k, seed=n)
    w = device_weight(sw)
    rows = rows_of(n, n + 1)
    w64 = rows_w64(sw, rows, row_indices(sw, rows))
    xs, x64 = vqsynth.make_x(1, k, "bf16", np.random.SeedSequence(n + 2))
    y = vq.vq_gemv(w, x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(w64, x64)
    assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"max 16-bit {kernel}")


@pytest.mark.parametrize("m,path", [(524272, "fp16"), (524287, "bf16")])
def test_max_tokens_gemm(vq, m, path):
    """m * k_in just below 2^31 on a 4096 x 4096 weight: at m = 524272 the
    fp16 path's padded x (2 m k bytes) just fits its 32-bit buffer; at
    524287 the padding (m rounded up to 16) would reach 2^31 elements and
    the call takes the bf16 path.  x is a block of 4093 seeded tokens
    repeated (4093 divides neither 2^18 nor 2^19, so a read that wraps by
    2^31 or 2^32 bytes lands on another token); y is checked on sampled
    tokens, the first and last ones included."""
    import torch
    n, k, blk = 4096, 4096, 4093
    assert m * k < LIMIT and m * n < LIMIT
    print(f"max tokens gemm m={m} ({path})", flush=True)
    sw = vqsynth.random_weight(n, k, 2, 12, 128, seed=6)
    w = device_weight(sw)
    assert (vq.vq_gemm_workspace_size(w, m) > 0) == (path == "fp16")
    xs, x64 = vqsynth.make_x(blk, k, "bf16", np.random.SeedSequence(m))
    x = x_to_device(xs, "bf16").repeat((m + blk - 1) // blk, 1)[:m]
    y = vq.vq_gemm(w, x)
    toks = rows_of(m, m + 1, count=64)
    got = y[torch.from_numpy(toks).cuda()].cpu().numpy()
    del x, y
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64[toks % blk])
    assert_within(got, y_ref, bound, f"gemm m={m}")
