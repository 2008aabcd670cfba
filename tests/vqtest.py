"""Test helpers: move synthetic weights to the device and build oracle
references for the same inputs.  The oracle and the HIP library only meet
here, in the tests."""
from __future__ import annotations

import os

import numpy as np

import oracle
import vqsynth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ensure_built():
    """Build the library if no built copy exists (tests load what is built)."""
    from compressed_index_matmul_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from compressed_index_matmul_amd.build import build
        build()


def device_weight(sw: vqsynth.SynthWeight, device="cuda"):
    from compressed_index_matmul_amd import VQWeight
    return VQWeight(sw.n_out, sw.k_in, sw.n_stages, sw.idx_bits, sw.scale_block,
                    codebooks=sw.codebooks, scales=sw.scales, lo=sw.lo, hi=sw.hi,
                    idx16=sw.idx16, device=device, stage_bits=sw.stage_bits,
                    stage_scales=sw.stage_scales, sparse=sw.sparse, lowrank=sw.lowrank)


def sparse_rows(sw: vqsynth.SynthWeight, rows):
    """The sparse correction restricted to `rows` (None: all), as CSR."""
    if sw.sparse is None or rows is None:
        return sw.sparse
    rp, cl, vl = sw.sparse
    parts_c, parts_v, ptr = [], [], [0]
    for r in rows:
        parts_c.append(cl[rp[r]:rp[r + 1]])
        parts_v.append(vl[rp[r]:rp[r + 1]])
        ptr.append(ptr[-1] + rp[r + 1] - rp[r])
    return (np.array(ptr), np.concatenate(parts_c) if parts_c else np.zeros(0, np.int64),
            np.concatenate(parts_v) if parts_v else np.zeros(0, np.float16))


def lowrank_rows(sw: vqsynth.SynthWeight, rows):
    """The low-rank factors restricted to `rows` of U (None: all)."""
    if sw.lowrank is None or rows is None:
        return sw.lowrank
    u, v = sw.lowrank
    return u[np.asarray(rows)], v


def product_ref(sw: vqsynth.SynthWeight, x64, rows=None, idx=None):
    """(y_ref, bound) of x against the selected rows: the oracle's exact
    product and its acceptance scale, with the low-rank correction's
    factor-wise scale added when the weight has one."""
    y_ref, bound = oracle.matmul_ref(oracle_w64(sw, rows, idx), x64)
    lr = lowrank_rows(sw, rows)
    if lr is not None:
        bound = bound + oracle.lowrank_bound(x64, lr)
    return y_ref, bound


def oracle_indices(sw: vqsynth.SynthWeight):
    return [oracle.unpack_indices(b, sw.n_groups, lo=sw.lo[t], hi=sw.hi[t], idx16=sw.idx16[t])
            for t, b in enumerate(sw.widths)]


def oracle_w64(sw: vqsynth.SynthWeight, rows=None, idx=None):
    """Exact float64 dequant of the selected rows (all rows if None)."""
    idx = oracle_indices(sw) if idx is None else idx
    g = sw.k_in // 8
    if rows is None:
        return oracle.dequant_exact(sw.n_out, sw.k_in, idx, sw.codebooks, sw.scales, sw.scale_block,
                                    sw.stage_scales, sw.sparse, sw.lowrank)
    rows = np.asarray(rows)
    sub = [i.reshape(sw.n_out, g)[rows].reshape(-1) for i in idx]
    return oracle.dequant_exact(len(rows), sw.k_in, sub, sw.codebooks, sw.scales[rows], sw.scale_block,
                                sw.stage_scales, sparse_rows(sw, rows), lowrank_rows(sw, rows))


def oracle_w16(sw: vqsynth.SynthWeight, rows=None, idx=None):
    idx = oracle_indices(sw) if idx is None else idx
    g = sw.k_in // 8
    if rows is None:
        return oracle.dequant_fp16(sw.n_out, sw.k_in, idx, sw.codebooks, sw.scales, sw.scale_block,
                                   sw.stage_scales, sw.sparse, sw.lowrank)
    rows = np.asarray(rows)
    sub = [i.reshape(sw.n_out, g)[rows].reshape(-1) for i in idx]
    return oracle.dequant_fp16(len(rows), sw.k_in, sub, sw.codebooks, sw.scales[rows], sw.scale_block,
                               sw.stage_scales, sparse_rows(sw, rows), lowrank_rows(sw, rows))


def sample_rows(n: int, count: int, seed: int):
    """First, last and `count` random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    r = set(rng.choice(n, size=min(count, n), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(r))


def x_to_device(x_stored, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x_stored).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_stored, dtype=np.float32)).to(device)


def assert_within(y, y_ref, bound, what=""):
    ok, worst = oracle.within_tolerance(y, y_ref, bound)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} outputs outside the bound "
                             f"(worst ratio {worst:.3g}); first {bad.tolist()}")
    return worst


def assert_all_rows(y, sw: vqsynth.SynthWeight, x64, what="", chunk=4096):
    """Every output of y [B, n_out] against the oracle's exact product, the
    float64 weight built a block of rows at a time to bound host memory."""
    idx = oracle_indices(sw)
    worst = 0.0
    for r0 in range(0, sw.n_out, chunk):
        rows = np.arange(r0, min(r0 + chunk, sw.n_out))
        y_ref, bound = product_ref(sw, x64, rows, idx)
        worst = max(worst, assert_within(y[:, rows], y_ref, bound, f"{what} rows {r0}.."))
    return worst
