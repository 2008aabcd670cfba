"""Parity of residual ladders (per-stage index widths) and per-stage residual
scales with the CPU oracle, through the C ABI.

Formats: orka's rvq-12-4 (a 12-bit primary plus a 4-bit residual stage),
GLQ's bit-width ladders (a 16-bit primary with 8- and 16-bit residual
stages, "Bit widths"), and the inverse residual scale of GLQ's two-stage
call ("Inference kernels").  Bars as everywhere: indices and the fp16
dequant bit for bit (with stage scales, the oracle's fixed float64
evaluation order), products within |y - y_ref| <= 2e-3 sum|w x| + 1e-6.
"""
import json
import os

import numpy as np
import pytest

import oracle
import vqsynth
from conftest import GOLDEN
from vqtest import (assert_within, device_weight, ensure_built, oracle_indices, oracle_w16, oracle_w64,
                    sample_rows, x_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


# (widths, stage-scale range or None): the LDS-kernel ladders (12+4, 8+4,
# 1-2 stages of 8/12 bits with scales) and the general-kernel ones
FORMATS = [
    ((12, 4), None), ((12, 4), (0.2, 0.4)), ((8, 4), None), ((8, 4), (0.5, 2.0)),
    ((12,), (0.5, 2.0)), ((12, 12), (0.2, 0.4)), ((8, 8), (-2.0, -0.5)),
    ((16, 8), (0.2, 0.4)), ((16, 16), None), ((16, 16, 8), (0.2, 0.4)), ((4,), None),
    ((12, 12, 4), None), ((16, 12, 8, 4), (0.3, 0.6)), ((8, 8, 8), (0.2, 0.4)),
]


def fmt_id(f):
    w, r = f
    return "+".join(map(str, w)) + ("/rs" if r else "")


def make(widths, rs, n, k, bs, seed, first_scale=None):
    sd = (0.02,) + tuple(0.02 * (0.3 if rs is None else 1.0) for _ in widths[1:])
    sw = vqsynth.random_weight(n, k, len(widths), list(widths), bs, seed, cb_sd=sd, stage_scale_range=rs)
    if first_scale is not None and sw.stage_scales is not None:
        sw.stage_scales[0] = np.float32(first_scale)
    return sw


def check_dequant(vq, sw, what):
    import torch
    w = device_weight(sw)
    idx_d, w_d = vq.vq_unpack_dequant(w)
    torch.cuda.synchronize()
    idx = oracle_indices(sw)
    got_idx = idx_d.cpu().numpy().view(np.uint16).reshape(sw.n_stages, -1)
    for t in range(sw.n_stages):
        assert np.array_equal(got_idx[t].astype(np.int64), idx[t]), f"{what}: stage {t} indices"
    want = oracle_w16(sw, None, idx)
    assert np.array_equal(w_d.cpu().numpy().view(np.uint16), want.view(np.uint16)), f"{what}: fp16 weights"


@pytest.mark.parametrize("fmt", FORMATS, ids=fmt_id)
@pytest.mark.parametrize("shape", [(37, 264, 24), (300, 1024, 128)], ids=["ragged", "tiles"])
def test_ladder_dequant_bitexact(vq, fmt, shape):
    n, k, bs = shape
    widths, rs = fmt
    sw = make(widths, rs, n, k, bs, seed=11 + len(widths), first_scale=1.25 if rs else None)
    check_dequant(vq, sw, f"{fmt_id(fmt)} {shape}")


def test_dequant_fixed_order_tie(vq):
    """The golden tie: float64 stage-order evaluation drops 2^-60 and the
    fp16 rounding of the exact fp64 tie goes to even (0x3C00)."""
    import torch
    from compressed_index_matmul_amd import VQWeight
    with open(os.path.join(GOLDEN, "stage_scale_hand.json")) as f:
        case = [c for c in json.load(f)["cases"] if "w_bits" in c][0]
    cbs = []
    for spec in case["codebooks_sparse"]:
        cb = np.zeros((spec["rows"], 8), np.float16)
        for row, vals in spec["set"].items():
            cb[int(row)] = vals
        cbs.append(cb)
    lo = [np.array(i, np.uint8) for i in case["indices"]]
    w = VQWeight(1, 8, 2, 8, 8, codebooks=cbs, scales=np.array(case["scales"], np.float16), lo=lo,
                 hi=[None, None], idx16=[None, None], stage_scales=case["stage_scales"])
    _, w_d = vq.vq_unpack_dequant(w, want_idx=False)
    torch.cuda.synchronize()
    assert w_d.cpu().numpy().view(np.uint16).tolist() == case["w_bits"]


@pytest.mark.parametrize("fmt", FORMATS, ids=fmt_id)
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(37, 264, 24), (700, 2048, 128), (129, 6144, 128)],
                         ids=["ragged", "lds", "long"])
def test_ladder_gemv(vq, fmt, xdt, shape):
    import torch
    n, k, bs = shape
    widths, rs = fmt
    sw = make(widths, rs, n, k, bs, seed=31 + k, first_scale=0.75 if rs else None)
    xs, x64 = vqsynth.make_x(1, k, xdt, np.random.SeedSequence(7 + n))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, xdt))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"{fmt_id(fmt)} {shape} {xdt}")


@pytest.mark.parametrize("fmt", [((12, 4), None), ((12, 4), (0.2, 0.4)), ((12, 12), (0.2, 0.4)), ((8, 4), None),
                                 ((16, 8), (0.2, 0.4)), ((8, 8), (0.5, 1.5))], ids=fmt_id)
@pytest.mark.parametrize("batch", [2, 3, 4, 7, 16])
def test_ladder_gemv_tokens(vq, fmt, batch):
    """2..4 bf16 tokens on the LDS kernel where instantiated, the rest on
    matrix cores; every token against the oracle."""
    import torch
    widths, rs = fmt
    n, k, bs = 520, 4096, 128
    sw = make(widths, rs, n, k, bs, seed=53 + batch)
    xs, x64 = vqsynth.make_x(batch, k, "bf16", np.random.SeedSequence(99 + batch))
    y = vq.vq_gemv(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"{fmt_id(fmt)} B={batch}")


@pytest.mark.parametrize("fmt", [((12, 4), None), ((12, 12), (0.2, 0.4)), ((16, 8), (0.2, 0.4)),
                                 ((16, 16, 8), None), ((8, 4), (0.5, 1.5))], ids=fmt_id)
@pytest.mark.parametrize("m", [1, 16, 17, 300])
def test_ladder_gemm(vq, fmt, m):
    import torch
    widths, rs = fmt
    n, k, bs = 333, 1032, 24   # ragged N, K not a multiple of 32, 24-column scale blocks
    sw = make(widths, rs, n, k, bs, seed=71 + m)
    xs, x64 = vqsynth.make_x(m, k, "bf16", np.random.SeedSequence(5 + m))
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw), x64)
    assert_within(y.cpu().numpy(), y_ref, bound, f"{fmt_id(fmt)} m={m}")


@pytest.mark.parametrize("m", [16, 64, 512])
def test_ladder_gemm_aligned(vq, m):
    """12+4 at an aligned Llama-like shape (K % 256 == 0, 128-column blocks)."""
    import torch
    sw = make((12, 4), None, 1000, 4096, 128, seed=3)
    xs, x64 = vqsynth.make_x(m, 4096, "bf16", np.random.SeedSequence(m))
    y = vq.vq_gemm(device_weight(sw), x_to_device(xs, "bf16"))
    torch.cuda.synchronize()
    rows = sample_rows(1000, 64, m)
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), x64)
    assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"12+4 m={m}")


# ---------------------------------------------------------------------------
# the ladder workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wl", ["smollm_rvq124", "llama8b_rvq124", "mlp70b_e8p3"])
def test_ladder_workload_dequant(vq, wl):
    import torch
    ws, _ = vqsynth.workload_weights(wl)
    for i, sw in enumerate(ws):
        w = device_weight(sw)
        idx_d, w_d = vq.vq_unpack_dequant(w)
        torch.cuda.synchronize()
        idx = oracle_indices(sw)
        got_idx = idx_d.cpu().numpy().view(np.uint16).reshape(sw.n_stages, -1)
        for t in range(sw.n_stages):
            assert np.array_equal(got_idx[t].astype(np.int64), idx[t]), f"{wl}/{sw.name} stage {t}"
        rows = None if sw.n_out * sw.k_in <= (1 << 22) else sample_rows(sw.n_out, 48, 100 + i)
        want = oracle_w16(sw, rows, idx)
        got = w_d.cpu().numpy()
        if rows is not None:
            got = got[rows]
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), f"{wl}/{sw.name} fp16"
        del w, idx_d, w_d


@pytest.mark.parametrize("wl", ["smollm_rvq124", "llama8b_rvq124"])
def test_ladder_workload_gemv(vq, wl):
    import torch
    ws, act_ss = vqsynth.workload_weights(wl)
    cfg = vqsynth.WORKLOADS[wl]
    kids = act_ss.spawn(2 * len(ws))
    for i, sw in enumerate(ws):
        w = device_weight(sw)
        rows = None if sw.n_out * sw.k_in <= (1 << 22) else sample_rows(sw.n_out, 48, 200 + i)
        w64 = oracle_w64(sw, rows)
        for b, kid in zip(cfg["batches"], (kids[i], kids[len(ws) + i])):
            xs, x64 = vqsynth.make_x(b, sw.k_in, cfg["x_dtype"], kid)
            y = vq.vq_gemv(w, x_to_device(xs, cfg["x_dtype"]))
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            if rows is not None:
                got = got[:, rows]
            y_ref, bound = oracle.matmul_ref(w64, x64)
            assert_within(got, y_ref, bound, f"{wl}/{sw.name} B={b}")


def test_ladder_workload_rht_gemv_mlp70b(vq):
    import torch
    ws, act_ss = vqsynth.workload_weights("mlp70b_e8p3")
    kids = act_ss.spawn(2 * len(ws))
    for i, sw in enumerate(ws):
        xs, x64 = vqsynth.make_x(1, sw.k_in, "bf16", kids[i])
        signs = vqsynth.make_signs(sw.k_in, kids[len(ws) + i])
        w = device_weight(sw)
        xr = vq.rht_apply(x_to_device(xs, "bf16"), torch.from_numpy(signs).cuda(), 8192)
        y = vq.vq_gemv(w, xr)
        torch.cuda.synchronize()
        rows = sample_rows(sw.n_out, 48, 400 + i)
        y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows), oracle.rht_ref(x64, signs, 8192))
        assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"mlp70b_e8p3/{sw.name}")


# shapes that route to each tuned matrix-core kernel: the 1..64-token unit
# kernel (N/16 units >= half the CUs, K % 256, 128-column scale blocks), the
# 256 x 128 tile kernel, and the 256 x 256 wide kernel (one tile per CU)
TUNED = {"few": (4096, 1024, 128, (1, 16, 17, 64)), "tile": (1000, 1024, 128, (300,)),
         "wide": (8192, 256, 128, (2048,))}


@pytest.mark.parametrize("fmt", [((12, 4), None), ((8, 4), (0.5, 1.5)), ((12, 4), (0.2, 0.4)), ((12, 12), (0.2, 0.4)),
                                 ((12,), (0.5, 2.0)), ((8, 8), (-2.0, -0.5))], ids=fmt_id)
@pytest.mark.parametrize("kern", list(TUNED))
def test_ladder_tuned_gemm_kernels(vq, fmt, kern):
    import torch
    widths, rs = fmt
    n, k, bs, ms = TUNED[kern]
    sw = make(widths, rs, n, k, bs, seed=97 + n, first_scale=1.5 if rs else None)
    w = device_weight(sw)
    rows = sample_rows(n, 64, 7)
    w64 = oracle_w64(sw, rows)
    for m in ms:
        xs, x64 = vqsynth.make_x(m, k, "bf16", np.random.SeedSequence(1000 + m))
        y = vq.vq_gemm(w, x_to_device(xs, "bf16"))
        torch.cuda.synchronize()
        y_ref, bound = oracle.matmul_ref(w64, x64)
        assert_within(y.cpu().numpy()[:, rows], y_ref, bound, f"{fmt_id(fmt)} {kern} m={m} sampled rows")
        if kern == "wide":  # every W row for a few tokens
            toks = sample_rows(m, 8, 3)
            y_ref2, bound2 = oracle.matmul_ref(oracle_w64(sw), x64[toks])
            assert_within(y.cpu().numpy()[toks], y_ref2, bound2, f"{fmt_id(fmt)} wide token rows")
