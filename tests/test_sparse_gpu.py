"""Parity of the sparse correction (orka README, "How it works": the decoded
weight plus a sparse correction) with the CPU oracle, through the C ABI.

The correction is CSR over output rows, added to the scaled decode.  Bars:
the fp16 dequant bit for bit (float64, entries in storage order, one
rounding); products within |y - y_ref| <= 2e-3 sum|w x| + 1e-6 with w the
corrected weight.
"""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import (assert_within, device_weight, ensure_built, oracle_indices, oracle_w16, oracle_w64,
                    sample_rows, x_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


# (widths, stage-scale range): a plain format, an LDS ladder, a general ladder
FORMATS = [((12, 12), None), ((12, 4), (0.2, 0.4)), ((16, 8), (0.2, 0.4)), ((8,), None)]


def fmt_id(f):
    return "+".join(map(str, f[0])) + ("/rs" if f[1] else "")


def make(fmt, n, k, bs, seed, density):
    widths, rs = fmt
    sd = (0.02,) + tuple(0.02 * (0.3 if rs is None else 1.0) for _ in widths[1:])
    return vqsynth.random_weight(n, k, len(widths), list(widths), bs, seed, cb_sd=sd, stage_scale_range=rs,
                                 sparse_density=density)


def with_duplicates(sw):
    """Give every third row a repeated column (entries stay ascending)."""
    rp, cl, vl = sw.sparse
    cl = cl.copy()
    for r in range(0, sw.n_out, 3):
        if rp[r + 1] - rp[r] >= 2:
            cl[rp[r] + 1] = cl[rp[r]]
    sw.sparse = (rp, cl, vl)
    return sw


@pytest.mark.parametrize("fmt", FORMATS, ids=fmt_id)
@pytest.mark.parametrize("shape", [(37, 264, 24), (300, 1024, 128)], ids=["ragged", "tiles"])
def test_sparse_dequant_bitexact(vq, fmt, shape):
    import torch
    n, k, bs = shape
    sw = with_duplicates(make(fmt, n, k, bs, 5 + n, 0.03))
    idx_d, w_d = vq.vq_unpack_dequant(device_weight(sw))
    torch.cuda.synchronize()
    idx = oracle_indices(sw)
    got_idx = idx_d.cpu().numpy().view(np.uint16).reshape(sw.n_stages, -1)
    for t in range(sw.n_stages):
        assert np.array_equal(got_idx[t].astype(np.int64), idx[t])
    want = oracle_w16(sw, None, idx)
    assert np.array_equal(w_d.cpu().numpy().view(np.uint16), want.view(np.uint16))


def test_sparse_dequant_empty_rows_and_cancel(vq):
    """Rows without entries, an entry cancelling its decoded weight to +0,
    and entries in the first and last column."""
    import torch
    sw = make(((12,), None), 6, 64, 64, 3, 0.05)
    w16 = oracle_w16(sw)
    rowptr = np.array([0, 0, 3, 3, 4, 4, 6])
    col = np.array([0, 17, 63, 5, 0, 63])
    val = np.array([0.5, -float(w16[1, 17]), 1.0, -2.0, 0.25, -0.125], np.float16)
    sw.sparse = (rowptr, col, val)
    _, w_d = vq.vq_unpack_dequant(device_weight(sw), want_idx=False)
    torch.cuda.synchronize()
    want = oracle_w16(sw)
    got = w_d.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    assert float(got[1, 17]) == 0.0 or got[1, 17] == want[1, 17]


@pytest.mark.parametrize("fmt", FORMATS, ids=fmt_id)
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("batch", [1, 3, 9])
def test_sparse_gemv(vq, fmt, xdt, batch):
    import torch
    sw = with_duplicates(make(fmt, 700, 2048, 128, 11, 0.01))
    xs, x64 = vqsynth.make_x(batch, 2048, xdt, np.random.SeedSequence(batch))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"{fmt_id(fmt)} {xdt} B={batch}")


@pytest.mark.parametrize("k,xdt", [(576, "bf16"), (4096, "bf16"), (4096, "f32"), (6144, "bf16")],
                         ids=["x-copied-per-lane", "x-lds-direct", "x-gathered-f32", "x-gathered-bf16"])
def test_sparse_mid_tokens(vq, k, xdt):
    """9-64 tokens on the separate correction kernel: x of the token block in
    LDS (copied by lanes when a row is not whole 1 KiB pieces, by LDS-direct
    loads when it is) or gathered from global memory (more than 8 KiB per
    token); 12 tokens, ragged against the 16-token block."""
    import torch
    sw = with_duplicates(make(((12, 12), None), 333, k, 64, 41 + k, 0.02))
    xs, x64 = vqsynth.make_x(12, k, xdt, np.random.SeedSequence(k))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"k={k} {xdt}")


def test_sparse_gemv_one_hot(vq):
    """x = e_c recovers the corrected column c (fp32 x, one token)."""
    import torch
    sw = make(((12, 12), None), 257, 1024, 128, 17, 0.02)
    w64 = oracle_w64(sw)
    w = device_weight(sw)
    for c in (0, int(sw.sparse[1][0]), 1023):
        x = np.zeros((1, 1024), np.float32)
        x[0, c] = 1.0
        y = vq.vq_gemv(w, torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        assert np.allclose(y.cpu().numpy()[0], w64[:, c], rtol=1e-6, atol=1e-7), c


@pytest.mark.parametrize("fmt", FORMATS, ids=fmt_id)
@pytest.mark.parametrize("m", [16, 40, 64, 300])
def test_sparse_gemm(vq, fmt, m):
    import torch
    sw = make(fmt, 4096, 1024, 128, 23, 0.01)
    xs, x64 = vqsynth.make_x(m, 1024, "bf16", np.random.SeedSequence(m))
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    rows = sample_rows(4096, 64, m)
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), x64)
    assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"{fmt_id(fmt)} m={m}")


def test_sparse_workload_llama8b(vq):
    """The Llama-3-8B linears with a 0.5 % correction: dequant (sampled rows)
    bit for bit, B=1 and B=16 products on sampled rows."""
    import torch
    ws, act_ss = vqsynth.workload_weights("llama8b_sparse")
    kids = act_ss.spawn(2 * len(ws))
    for i, sw in enumerate(ws):
        w = device_weight(sw)
        rows = sample_rows(sw.n_out, 48, 700 + i)
        _, w_d = vq.vq_unpack_dequant(w, want_idx=False)
        torch.cuda.synchronize()
        assert np.array_equal(w_d.cpu().numpy()[rows].view(np.uint16), oracle_w16(sw, rows).view(np.uint16))
        del w_d
        w64 = oracle_w64(sw, rows)
        for b, kid in zip((1, 16), (kids[i], kids[len(ws) + i])):
            xs, x64 = vqsynth.make_x(b, sw.k_in, "bf16", kid)
            y = vq.vq_gemv(w, x_to_device(xs, "bf16"))
            torch.cuda.synchronize()
            y_ref, bound = oracle.matmul_ref(w64, x64)
            assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"llama8b_sparse/{sw.name} B={b}")
