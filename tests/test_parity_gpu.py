"""Parity of the HIP path with the CPU oracle at the workloads' full sizes.

Indices and the fp16 dequant must match bit for bit; matmul outputs must lie
within |y - y_ref| <= 2e-3 * sum|w x| + 1e-6 of the exact float64 product;
the Hadamard transform within its fp32 forward-error bound.  Every output of
the decode products (one and sixteen tokens, the 70B MLP with its input
transform), every output of the 2048-token GEMM and every dequantized
weight is compared, the oracle's weight built a block of rows at a time.
"""
import numpy as np
import pytest

import oracle
import vqsynth
from vqtest import (assert_all_rows, assert_within, device_weight, ensure_built, oracle_indices, oracle_w16,
                    oracle_w64, x_to_device)

pytestmark = pytest.mark.gpu

_CACHE = {}


def workload(wl):
    if wl not in _CACHE:
        ws, act_ss = vqsynth.workload_weights(wl)
        _CACHE[wl] = (ws, act_ss)
    return _CACHE[wl]


@pytest.fixture(scope="module")
def vq():
    ensure_built()
    import compressed_index_matmul_amd as m
    m.lib()
    return m


def rht_bound(x64, signs, n, max_block):
    """Elementwise forward-error bound of an fp32 orthonormal FWHT, per block:
    (log2(nb) + 2) * 2^-24 * ||x_block||_2 * 1.01 (one rounding per butterfly
    stage plus the final scale and its rounded constant)."""
    out = np.empty_like(x64)
    off = 0
    for nb in oracle.rht_blocks(n, max_block):
        nrm = np.linalg.norm(x64[:, off:off + nb], axis=1, keepdims=True)
        out[:, off:off + nb] = (np.log2(nb) + 2) * 2.0 ** -24 * nrm * 1.01
        off += nb
    return out


@pytest.mark.parametrize("wl", ["tiny", "smollm", "llama8b", "mlp70b", "prefill"])
def test_unpack_dequant_bitexact(vq, wl):
    import torch
    ws, _ = workload(wl)
    for i, sw in enumerate(ws):
        w = device_weight(sw)
        idx_d, w_d = vq.vq_unpack_dequant(w)
        torch.cuda.synchronize()
        idx = oracle_indices(sw)
        got_idx = idx_d.cpu().numpy().view(np.uint16).reshape(sw.n_stages, -1)
        for t in range(sw.n_stages):
            assert np.array_equal(got_idx[t].astype(np.int64), idx[t]), f"{wl}/{sw.name} stage {t} indices"
        got = w_d.cpu().numpy().view(np.uint16)
        for r0 in range(0, sw.n_out, 4096):  # every weight, a block of rows at a time
            rows = np.arange(r0, min(r0 + 4096, sw.n_out))
            want = oracle_w16(sw, rows, idx)
            assert np.array_equal(got[rows], want.view(np.uint16)), f"{wl}/{sw.name} fp16 weights rows {r0}.."
        del w, idx_d, w_d


@pytest.mark.parametrize("wl", ["tiny", "smollm", "llama8b"])
def test_gemv_batch1(vq, wl):
    import torch
    ws, act_ss = workload(wl)
    cfg = vqsynth.WORKLOADS[wl]
    kids = act_ss.spawn(len(ws))
    for i, sw in enumerate(ws):
        xs, x64 = vqsynth.make_x(1, sw.k_in, cfg["x_dtype"], kids[i])
        w = device_weight(sw)
        y = vq.vq_gemv(w, x_to_device(xs, cfg["x_dtype"]))
        torch.cuda.synchronize()
        assert_all_rows(y.cpu().numpy(), sw, x64, f"{wl}/{sw.name}")


def test_gemv_batch16_llama8b(vq):
    import torch
    ws, act_ss = workload("llama8b")
    kids = act_ss.spawn(2 * len(ws))
    for i, sw in enumerate(ws):
        xs, x64 = vqsynth.make_x(16, sw.k_in, "bf16", kids[len(ws) + i])
        w = device_weight(sw)
        y = vq.vq_gemv(w, x_to_device(xs, "bf16"))
        torch.cuda.synchronize()
        assert_all_rows(y.cpu().numpy(), sw, x64, f"llama8b/{sw.name} B=16")


def test_rht_mlp70b_inputs(vq):
    import torch
    ws, act_ss = workload("mlp70b")
    kids = act_ss.spawn(2 * len(ws))
    for i, sw in enumerate(ws):
        xs, x64 = vqsynth.make_x(1, sw.k_in, "bf16", kids[i])
        signs = vqsynth.make_signs(sw.k_in, kids[len(ws) + i])
        xr = vq.rht_apply(x_to_device(xs, "bf16"), torch.from_numpy(signs).cuda(), 8192)
        torch.cuda.synchronize()
        ref = oracle.rht_ref(x64, signs, 8192)
        err = np.abs(xr.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= rht_bound(x64, signs, sw.k_in, 8192)), f"{sw.name}: max err {err.max()}"


def test_rht_gemv_mlp70b(vq):
    """Input transform then 16-bit-index GEMV (1 MiB codebook): the result is
    checked against the oracle's exact transform and exact product."""
    import torch
    ws, act_ss = workload("mlp70b")
    kids = act_ss.spawn(2 * len(ws))
    for i, sw in enumerate(ws):
        xs, x64 = vqsynth.make_x(1, sw.k_in, "bf16", kids[i])
        signs = vqsynth.make_signs(sw.k_in, kids[len(ws) + i])
        w = device_weight(sw)
        xr = vq.rht_apply(x_to_device(xs, "bf16"), torch.from_numpy(signs).cuda(), 8192)
        y = vq.vq_gemv(w, xr)
        torch.cuda.synchronize()
        xr_ref = oracle.rht_ref(x64, signs, 8192)
        assert_all_rows(y.cpu().numpy(), sw, xr_ref, f"mlp70b/{sw.name}")


def test_gemm_prefill(vq):
    """2048-token GEMM: every output against the oracle's exact product, the
    float64 weight built a block of rows at a time."""
    import torch
    ws, act_ss = workload("prefill")
    kids = act_ss.spawn(len(ws))
    for i, sw in enumerate(ws):
        print(f"prefill {sw.name} {sw.n_out}x{sw.k_in}", flush=True)
        xs, x64 = vqsynth.make_x(2048, sw.k_in, "bf16", kids[i])
        w = device_weight(sw)
        y = vq.vq_gemm(w, x_to_device(xs, "bf16"))
        torch.cuda.synchronize()
        assert_all_rows(y.cpu().numpy(), sw, x64, f"prefill/{sw.name}", chunk=2048)
        del w, y
