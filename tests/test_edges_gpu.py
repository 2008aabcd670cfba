"""Edge cases on the GPU: ragged shapes (partial tiles, odd group counts, short
last scale block), every index width and stage count, both activation types,
batch sizes 1..16, extreme fp16 values for the bit-exact dequant, ragged
GEMM, transform sizes, determinism and streams."""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import (assert_within, device_weight, ensure_built, oracle_indices, oracle_w16, oracle_w64, sample_rows,
                    x_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


# (n, k, stages, bits, scale_block)
SHAPES = [
    (1, 8, 1, 12, 8),          # a single group: odd count, padded high nibble
    (3, 24, 2, 12, 8),         # odd groups per row: rows start mid-byte in the hi plane
    (37, 72, 1, 12, 16),       # K % 32 != 0 -> general path
    (576, 576, 1, 12, 128),    # last scale block 64 columns (fast path)
    (100, 160, 3, 12, 32),     # three 12-bit stages: codebooks do not fit LDS
    (64, 96, 4, 8, 32),        # four 8-bit stages in LDS
    (130, 256, 2, 16, 64),     # two 16-bit stages
    (33, 16384, 2, 12, 128),   # eight chunks per lane on the fast path
    (17, 8200, 1, 12, 8),      # long ragged K, per-group scales
    (5, 40000, 1, 8, 40000),   # K beyond the LDS-staged x of the general path
    (256, 512, 1, 8, 512),     # the tiny workload's format
    (4097, 4096, 2, 12, 128),  # one row past a multiple of the grid
]


def _x(batch, k, dtype, seed):
    return vqsynth.make_x(batch, k, dtype, np.random.SeedSequence(seed))


def bf16_worst_case_bound(bound, k):
    """Guaranteed bound of the bf16 matrix-core paths: every weight is
    rounded to bf16 (8 significant bits: relative error <= 2^-8, plus 2^-23
    for the fp32 product rounded before it), x is exact, products are exact
    in fp32 and at most K of them are accumulated in fp32."""
    return (2.0 ** -8 + 2.0 ** -23 + k * 2.0 ** -24) * bound + 1e-6


def assert_bf16_path(y, y_ref, bound, k, what, m=None, few=False):
    """bf16 paths: the worst-case bound always; the 2e-3 bound once K is
    large enough for the per-weight rounding errors to average (K >= 256).
    With at most 16 tokens (m given), or up to 64 on the few-token unit
    kernel (few), the weights enter as bf16 hi + lo parts and the 2e-3 bound
    holds for any K."""
    if m is not None and (m <= 16 or (few and m <= 64)):
        assert_within(y, y_ref, bound, what)
        return
    err = np.abs(np.asarray(y, np.float64) - y_ref)
    assert np.all(err <= bf16_worst_case_bound(bound, k)), f"{what}: beyond the bf16 worst-case bound"
    if k >= 256:
        assert_within(y, y_ref, bound, what)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("batch", [1, 3])
def test_gemv_ragged(vq, shape, dtype, batch):
    import torch
    n, k, st, bits, bs = shape
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=n * 131 + k + st + bits)
    xs, x64 = _x(batch, k, dtype, n + k)
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, dtype))
    torch.cuda.synchronize()
    rows = None if n <= 600 else np.array([0, 1, 2, n // 2, n - 2, n - 1])
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), x64)
    got = y.cpu().numpy()
    got = got if rows is None else got[:, rows]
    if batch > 1 and dtype == "bf16":   # 2..16 bf16 tokens run on bf16 matrix cores
        assert_bf16_path(got, y_ref, bound, k, f"{shape} {dtype} B={batch}", m=batch)
    else:                               # fp32 decode: the 2e-3 bound for any input
        assert_within(got, y_ref, bound, f"{shape} {dtype} B={batch}")


@pytest.mark.parametrize("n,k,st,bits,bs,batch", [(300, 1024, 2, 12, 128, 2), (1000, 4096, 2, 12, 128, 3),
                                                   (777, 6144, 1, 12, 64, 2), (513, 2080, 2, 8, 32, 4),
                                                   (256, 4096, 2, 12, 4096, 4)])
def test_gemv_tokens_lds(vq, n, k, st, bits, bs, batch):
    """2-4 bf16 tokens on the LDS decode kernel (every gathered codebook
    vector multiplied with each token's x): one to three chunks per lane,
    a ragged last chunk set, ragged rows, 8- and 12-bit; the last shape does
    not fit the LDS with four tokens and takes the matrix-core path."""
    import torch
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=n + k + batch)
    xs, x64 = _x(batch, k, "bf16", 31 + n + batch)
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"{n}x{k} B={batch}")


def test_gemv_tokens_lds_one_hot(vq):
    """Each of three tokens is a different unit vector: the outputs are three
    dequantized columns, exact up to fp32 rounding (fp16 products path)."""
    import torch
    n, k = 300, 1024
    sw = vqsynth.random_weight(n, k, 2, 12, 128, seed=5)
    cols = [0, 517, k - 1]
    x64 = np.zeros((3, k))
    for t, c in enumerate(cols):
        x64[t, c] = 1.0
    xs = (x64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # 1.0 is exact in bf16
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    w64 = oracle_w64(sw)
    y_ref, bound = oracle.matmul_ref(w64, x64)
    assert np.array_equal(y_ref, w64[:, cols].T)
    assert_within(y.cpu().numpy(), y_ref, bound, "one-hot tokens")


@pytest.mark.parametrize("batch", [2, 5, 16])
def test_gemv_small_batch_mfma(vq, batch):
    import torch
    sw = vqsynth.random_weight(300, 1024, 2, 12, 128, seed=batch)
    xs, x64 = _x(batch, 1024, "bf16", 77 + batch)
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"B={batch}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_unpack_dequant_ragged(vq, shape):
    import torch
    n, k, st, bits, bs = shape
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=n + 7 * k)
    idx_d, w_d = vq.vq_unpack_dequant(device_weight(sw))
    torch.cuda.synchronize()
    idx = oracle_indices(sw)
    got = idx_d.cpu().numpy().view(np.uint16).reshape(st, -1)
    for t in range(st):
        assert np.array_equal(got[t].astype(np.int64), idx[t])
    assert np.array_equal(w_d.cpu().numpy().view(np.uint16), oracle_w16(sw, None, idx).view(np.uint16))


def _extreme_weight(seed, n=64, k=64, st=3, bits=8):
    rng = np.random.default_rng(seed)
    pool = np.array([0.0, -0.0, 6e-8, -6e-8, 1.2e-7, 3.1e-5, -6.1e-5, 1e-3, 0.5, -1.0, 3.0, 100.0, -2500.0,
                     30000.0, 65504.0, -65504.0, 0.333, 2.005859375], dtype=np.float16)
    sw = vqsynth.random_weight(n, k, st, bits, 16, seed=seed)
    sw.codebooks = [rng.choice(pool, ((1 << bits), 8)).astype(np.float16) for _ in range(st)]
    sw.scales = rng.choice(np.array([0.75, -2.0, 1.5, 6e-8, 1024.0, -0.0, 0.999], np.float16),
                           sw.scales.shape).astype(np.float16)
    return sw


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_dequant_extreme_values(vq, seed):
    """Subnormals, overflow to inf, signed zeros, negative scales, mixed
    magnitudes across three stages: every weight bit-exact."""
    import torch
    sw = _extreme_weight(seed)
    _, w_d = vq.vq_unpack_dequant(device_weight(sw), want_idx=False)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):
        want = oracle_w16(sw)
    assert np.array_equal(w_d.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("bits,st", [(8, 2), (12, 1), (8, 4)])
def test_dequant_random_bit_patterns(vq, bits, st):
    """Codebooks and scales drawn as random finite fp16 bit patterns (every
    exponent, subnormals, both signs), so the single rounding of the exact
    value meets ties, subnormal results and overflow in bulk: every weight
    bit-exact."""
    import torch
    rng = np.random.default_rng(bits * 10 + st)

    def finite_bits(shape):
        b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
        b[(b & 0x7c00) == 0x7c00] &= 0xbfff  # inf / NaN exponents -> a finite one
        return b.view(np.float16)

    sw = vqsynth.random_weight(512, 256, st, bits, 32, seed=bits + st)
    sw.codebooks = [finite_bits(((1 << bits), 8)) for _ in range(st)]
    sw.scales = finite_bits(sw.scales.shape)
    _, w_d = vq.vq_unpack_dequant(device_weight(sw), want_idx=False)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):
        want = oracle_w16(sw)
    assert np.array_equal(w_d.cpu().numpy().view(np.uint16), want.view(np.uint16))


def test_dequant_double_rounding_trap(vq):
    """The hand-derived trap (s=0.75, cb0=2+3*2^-9, cb1=2^-24) rounds once."""
    import json
    import os
    import torch
    from conftest import GOLDEN
    d = json.load(open(os.path.join(GOLDEN, "double_rounding.json")))
    sw = vqsynth.random_weight(4, 64, 2, 8, 64, seed=9)
    sw.codebooks[0][:] = d["c0"]
    sw.codebooks[1][:] = d["c1"]
    sw.scales[:] = d["scale"]
    _, w_d = vq.vq_unpack_dequant(device_weight(sw), want_idx=False)
    torch.cuda.synchronize()
    assert np.all(w_d.cpu().numpy().view(np.uint16) == d["w_fp16_bits"])


@pytest.mark.parametrize("m,n,k,st,bits", [(17, 130, 72, 2, 12), (300, 257, 256, 1, 12), (1, 64, 4096, 2, 12),
                                          (40, 96, 8, 1, 8), (33, 200, 512, 1, 16), (513, 129, 160, 3, 12)])
def test_gemm_ragged(vq, m, n, k, st, bits):
    import torch
    sw = vqsynth.random_weight(n, k, st, bits, 8 if k % 32 else 32, seed=m + n + k)
    xs, x64 = _x(m, k, "bf16", m * 7 + n)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_bf16_path(y.cpu().numpy(), y_ref, bound, k, f"gemm {m}x{n}x{k}", m=m)


@pytest.mark.parametrize("m,n,k,st,bits,bs", [(257, 131, 512, 2, 12, 128), (40, 64, 768, 2, 8, 768),
                                             (18, 300, 256, 1, 12, 64), (600, 70, 1024, 2, 12, 1024),
                                             (300, 129, 2048, 2, 12, 32), (1300, 11000, 256, 2, 12, 128),
                                             (1100, 15000, 512, 1, 8, 64)])
def test_gemm_tile_ragged(vq, m, n, k, st, bits, bs):
    """Shapes of the large-M buffer-load kernel (K % 256 == 0): ragged token
    and W-row tiles, several scale-block sizes (one per K step up to one per
    row), 8- and 12-bit indices."""
    import torch
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=m * 3 + n + k + bs)
    xs, x64 = _x(m, k, "bf16", m * 11 + n)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_bf16_path(y.cpu().numpy(), y_ref, bound, k, f"gemm {m}x{n}x{k} bs {bs}", m=m)


@pytest.mark.parametrize("m,n,k,st,bits,bs", [(1900, 14300, 512, 2, 12, 128), (2048, 14336, 256, 2, 12, 128),
                                             (2048, 8192, 256, 2, 12, 256), (1800, 12000, 512, 1, 8, 64)])
def test_gemm_wide_row_tiles(vq, m, n, k, st, bits, bs):
    """The 256 x 256 wide kernel at its large shapes: a partly filled last
    round of tiles (14300, 14336 and 12000 rows at 8 token panels), one full
    round (8192 rows), ragged tokens and rows; sampled output columns
    (tile edges included) against the oracle."""
    import torch
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=m + n + k)
    xs, x64 = _x(m, k, "bf16", m * 5 + n)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(n, 96, n), [0, 223, 224, 255, 256, n - 1]]))
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), x64)
    assert_bf16_path(y.cpu().numpy()[:, rows], y_ref, bound, k, f"gemm {m}x{n}x{k} bs {bs}")


@pytest.mark.parametrize("m,n,k,st,bits,bs", [(2048, 8212, 256, 3, 8, 128), (1950, 8192, 512, 4, 8, 256)])
def test_gemm_wide_bf16_every_output(vq, m, n, k, st, bits, bs):
    """The bf16 256 x 256 wide kernel (three and four 8-bit stages, which have
    no fp16 variant) on every output: every one of a wave's 64 accumulator
    blocks in full tiles, a ragged last row tile and (second case) a ragged
    token panel, so a missing wait after the asm MFMAs shows up in any
    block."""
    import torch
    print(f"wide bf16 {m}x{n}x{k} stages {st}", flush=True)
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=m + n + st)
    xs, x64 = _x(m, k, "bf16", m * 7 + n)
    w = device_weight(sw)
    assert vq.vq_gemm_workspace_size(w, m) == 0, "three or more stages: the bf16 path"
    y = vq.vq_gemm(w, x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_bf16_path(y.cpu().numpy(), y_ref, bound, k, f"wide bf16 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k,st,bits,bs", [(17, 4096, 512, 2, 12, 128), (40, 8200, 1024, 1, 8, 1024),
                                             (64, 4100, 256, 2, 12, 256), (33, 2500, 768, 2, 12, 384),
                                             (16, 4096, 512, 1, 12, 128), (2, 2049, 512, 2, 12, 512)])
def test_gemm_token_blocks(vq, m, n, k, st, bits, bs):
    """Up to 64 tokens on the unit kernel: one to four 16-token blocks, one
    16-row block per unit (every CU busy from 128 units), ragged W rows and
    tokens, K parts of one to several trips, scale blocks of 128 columns up
    to a whole row."""
    import torch
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=m * 17 + n + k)
    xs, x64 = _x(m, k, "bf16", m * 19 + n)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_bf16_path(y.cpu().numpy(), y_ref, bound, k, f"gemm {m}x{n}x{k} bs {bs}", m=m, few=True)


@pytest.mark.parametrize("m,n,k,st,bits,bs", [(5, 8200, 512, 2, 12, 128), (16, 8192, 1024, 1, 8, 1024),
                                             (1, 9000, 256, 2, 12, 32), (11, 12000, 768, 2, 12, 64)])
def test_gemm_few_tokens_wide(vq, m, n, k, st, bits, bs):
    """Few tokens against wide weights (at least one 32-row unit per CU): the
    unit kernel with its K split across waves and the fixed-order partial
    sums, ragged W rows, 1-16 tokens, several scale blocks."""
    import torch
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=m * 5 + n + k)
    xs, x64 = _x(m, k, "bf16", m * 13 + n)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_bf16_path(y.cpu().numpy(), y_ref, bound, k, f"gemm {m}x{n}x{k} bs {bs}", m=m)


# (n, k, stages, widths, scale block, stage scales): the unit kernel (12+12,
# 8-bit), the slab kernel (16-bit), the general slab kernel (K % 128 != 0),
# a 12+4 ladder with stage scales, three 8-bit stages
ONE_HOT_SHAPES = [(2048, 1024, 2, 12, 128, None), (2304, 2048, 1, 8, 2048, None), (300, 1024, 1, 16, 1024, None),
                  (200, 520, 2, 12, 40, None), (1024, 768, 2, [12, 4], 128, (0.5, 1.5)),
                  (600, 512, 3, 8, 128, None)]


@pytest.mark.parametrize("shape", ONE_HOT_SHAPES, ids=lambda s: "x".join(str(v) for v in s[:4]))
@pytest.mark.parametrize("batch", [5, 8, 16])
def test_gemv_tokens_any_x(vq, shape, batch):
    """5-16 bf16 tokens on the matrix-core kernels meet the 2e-3 bound for
    any x: one-hot tokens, a token with one large and many tiny entries,
    sparse and dense tokens in one batch, every output against the oracle
    (bf16 weights alone would miss it on the one-hot tokens)."""
    import torch
    n, k, st, bits, bs, ssr = shape
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=n + k + batch, stage_scale_range=ssr)
    xs, x64 = _mixed_tokens(batch, k, batch * 7 + k)
    w = device_weight(sw)
    y = vq.vq_gemv(w, x_to_device(xs, "bf16"))
    y2 = vq.vq_gemm(w, x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"gemv {n}x{k} B={batch}")
    assert_within(y2.cpu().numpy(), y_ref, bound, f"gemm {n}x{k} m={batch}")


def _mixed_tokens(m, k, seed):
    """bf16 tokens of four kinds in turn: one-hot, one large entry over tiny
    ones, five nonzero columns, dense N(0,1)."""
    rng = np.random.default_rng(seed)
    x = np.zeros((m, k), np.float32)
    for b in range(m):
        kind = b % 4
        if kind == 0:
            x[b, rng.integers(k)] = 1.0
        elif kind == 1:
            x[b, :] = rng.standard_normal(k) * 2.0 ** -20
            x[b, rng.integers(k)] = 3.0
        elif kind == 2:
            cols = rng.choice(k, 5, replace=False)
            x[b, cols] = rng.standard_normal(5)
        else:
            x[b, :] = rng.standard_normal(k)
    xs = vqsynth.f32_to_bf16_bits(x)
    return xs, vqsynth.bf16_bits_to_f32(xs).astype(np.float64)


# (n, k, stages, widths, scale block, stage scales) on the few-token unit
# kernel (K % 256 == 0, scale blocks of 128 columns or more; with more than
# 16 tokens any row count up to eight 16-row units per CU): 12+12, one 8-bit
# stage, a 12+4 ladder with stage scales, three 8-bit stages, and row counts
# that leave most CUs idle (64, 13 and one unit, ragged)
FEW_SHAPES = [(2048, 1024, 2, 12, 128, None), (2304, 2048, 1, 8, 2048, None), (2064, 768, 2, [12, 4], 128, (0.5, 1.5)),
              (2176, 512, 3, 8, 128, None), (1024, 4096, 2, 12, 128, None), (200, 512, 1, 8, 128, None),
              (9, 256, 2, 12, 256, None)]


@pytest.mark.parametrize("shape", FEW_SHAPES, ids=lambda s: "x".join(str(v) for v in s[:4]))
@pytest.mark.parametrize("m", [17, 40, 64])
def test_gemm_tokens_any_x(vq, shape, m):
    """17-64 bf16 tokens on the few-token unit kernel (two to four token
    blocks) meet the 2e-3 bound for any x: one-hot, wide-range, sparse and
    dense tokens, every output against the oracle (bf16 weights alone miss
    it on the one-hot tokens)."""
    import torch
    n, k, st, bits, bs, ssr = shape
    sw = vqsynth.random_weight(n, k, st, bits, bs, seed=n + k + m, stage_scale_range=ssr)
    xs, x64 = _mixed_tokens(m, k, m * 11 + k)
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"gemm {n}x{k} m={m}")


def test_gemv_one_hot_columns(vq):
    """x = e_k through the fp32-decode path recovers dequantized columns to
    fp32 rounding (the oracle's one-hot pin, on the GPU)."""
    import torch
    sw = vqsynth.random_weight(512, 1024, 2, 12, 128, seed=31)
    w64 = oracle_w64(sw)
    w = device_weight(sw)
    for col in (0, 7, 8, 511, 1023):
        x = torch.zeros((1, 1024), dtype=torch.float32, device="cuda")
        x[0, col] = 1.0
        y = vq.vq_gemv(w, x)
        torch.cuda.synchronize()
        assert np.allclose(y.cpu().numpy()[0], w64[:, col], rtol=2.0 ** -22, atol=0)


@pytest.mark.parametrize("n,max_block", [(1, 8192), (2, 8192), (3, 8192), (2688, 8192), (28672, 16384),
                                         (28672, 8192), (100, 1), (4096, 64), (8192, 256), (8192, 512),
                                         (2560, 2048), (6144, 4096), (16384, 16384), (256, 8192)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rht_sizes(vq, n, max_block, dtype):
    import torch
    from test_parity_gpu import rht_bound
    xs, x64 = _x(3, n, dtype, n + max_block)
    signs = vqsynth.make_signs(n, np.random.SeedSequence(n))
    out = vq.rht_apply(x_to_device(xs, dtype), torch.from_numpy(signs).cuda(), max_block)
    torch.cuda.synchronize()
    ref = oracle.rht_ref(x64, signs, max_block)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= rht_bound(x64, signs, n, max_block)), err.max()


def test_deterministic_and_stream_independent(vq):
    """Bitwise-identical results on rerun and on a non-default stream (fixed
    reduction order, no atomics)."""
    import torch
    cases = [(vqsynth.random_weight(4096, 4096, 2, 12, 128, seed=5), "gemv", 1),
             (vqsynth.random_weight(1000, 2048, 1, 16, 2048, seed=6), "gemv", 1),
             (vqsynth.random_weight(700, 1024, 2, 12, 128, seed=7), "gemv", 16),
             (vqsynth.random_weight(640, 512, 2, 12, 128, seed=8), "gemm", 600)]
    for sw, op, b in cases:
        w = device_weight(sw)
        xs, _ = _x(b, sw.k_in, "bf16", b)
        x = x_to_device(xs, "bf16")
        f = vq.vq_gemv if op == "gemv" else vq.vq_gemm
        y1 = f(w, x)
        y2 = f(w, x)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            y3 = f(w, x, stream=s)
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(y1, y3), op


def test_concurrent_streams(vq):
    """Different products enqueued alternately on two streams with no
    synchronisation between them (each vq_gemm with its own workspace) give
    bit for bit the results of the same calls run one after another: the
    library keeps no state between calls except vq_gemm_noalloc's scratch."""
    import torch
    ws = [device_weight(vqsynth.random_weight(4096, 4096, 2, 12, 128, seed=11)),
          device_weight(vqsynth.random_weight(2048, 8192, 1, 16, 8192, seed=12)),
          device_weight(vqsynth.random_weight(4096, 1024, 2, [12, 4], 128, seed=13, stage_scale_range=(0.2, 0.4)))]
    xs = [x_to_device(_x(m, w.k_in, "bf16", 20 + i)[0], "bf16") for i, (w, m) in enumerate(zip(ws, (1, 1, 300)))]
    signs = torch.from_numpy(vqsynth.make_signs(8192, np.random.SeedSequence(21))).cuda()

    def calls(stream, wsp):
        return [lambda: vq.vq_gemv(ws[0], xs[0], stream=stream),
                lambda: vq.vq_gemv(ws[1], vq.rht_apply(xs[1], signs, 2048, stream=stream), stream=stream),
                lambda: vq.vq_gemm(ws[2], xs[2], workspace=wsp, stream=stream)]

    need = vq.vq_gemm_workspace_size(ws[2], 300)
    wsp = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    serial = [f() for f in calls(None, wsp[0])]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(4):
        for s, wp in ((s1, wsp[0]), (s2, wsp[1])):
            with torch.cuda.stream(s):
                outs.append([f() for f in calls(s, wp)])
    torch.cuda.synchronize()
    for got in outs:
        for a, b in zip(serial, got):
            assert torch.equal(a, b)
