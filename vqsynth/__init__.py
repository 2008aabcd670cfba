"""Seeded synthetic inputs for the compressed-index matmul.

This module only draws random numbers and lays them out in the storage
format; it holds none of the decode arithmetic.  Both the HIP library's tests
and the CPU oracle consume what it produces, so it imports neither.

Index planes are drawn directly as random bytes: a uniform 12-bit index is a
uniform low byte and an independent uniform high nibble, so the ``lo`` plane
is uniform bytes and the ``hi`` plane is uniform bytes (two nibbles per byte;
the pad nibble of an odd group count is cleared).  16-bit indices are uniform
uint16.  Codebooks are normal with the stated standard deviation rounded to
fp16; scales are uniform on [0.5, 1.5) rounded to fp16; activations are
standard normal rounded to bf16 (or kept fp32).

Workloads (one entry per weight format; shapes are nn.Linear [out, in]):

* ``tiny``      256x512, 1 stage, 8-bit indices, 256-entry codebook, one
                scale per row, fp32 x, batch 1.
* ``smollm``    SmolLM-135M linears (d=576, ffn=1536): q/k/v/o 576x576,
                gate/up 1536x576, down 576x1536; 1 stage, 12-bit bit-planes,
                4096-entry codebook, per-row x 128-column scales, bf16 x.
* ``llama8b``   Llama-3-8B-shaped linears 4096x4096, 14336x4096, 4096x14336;
                2 stages (12+12 bit), stage-2 codebook std 0.3x stage 1,
                per-row x 128-column scales, bf16 x, batch 1 and 16.
* ``mlp70b``    70B-MLP-shaped linears 28672x8192 and 8192x28672; 1 stage of
                16-bit indices into a 65,536-entry codebook, one scale per row,
                random +/-1 signs for the input Hadamard transform, bf16 x.
* ``prefill``   2048 tokens x (4096x4096, 14336x4096) in the llama8b format.

Residual ladders (per-stage index widths; optional per-stage residual
scales, drawn after everything else so the formats above are unchanged):

* ``smollm_rvq124``  SmolLM-135M linears in orka's rvq-12-4 mode: a 12-bit
                     stage (4096 entries) plus a 4-bit stage (16 entries,
                     std 0.3x), 2 bits per weight of indices.
* ``llama8b_rvq124`` the Llama-3-8B linears in the same 12+4 format.
* ``llama8b_sparse`` the llama8b format plus a sparse correction of 0.5 %
                     of each row's weights (values N(0, 0.05), fp16).
* ``llama8b_lowrank`` the llama8b format plus a rank-32 low-rank
                     correction U V (fp16 factors, see make_weight).
* ``mlp70b_e8p3``    the 70B-MLP linears as GLQ's 3 bpw ladder: a 16-bit
                     primary and an 8-bit residual stage whose codebook has
                     the primary's spread, brought down by a residual scale
                     drawn from U(0.2, 0.4); input transform as mlp70b.
* ``mlp70b_e8p4``    the same with a 16-bit residual stage (GLQ's 4 bpw ladder).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = ["SynthWeight", "WORKLOADS", "make_weight", "make_x", "make_signs",
           "workload_weights", "bf16_bits_to_f32"]


@dataclass
class SynthWeight:
    name: str
    n_out: int
    k_in: int
    n_stages: int
    idx_bits: int                     # stage 0's width (every stage's for a uniform ladder)
    scale_block: int
    lo: List[Optional[np.ndarray]] = field(default_factory=list)
    hi: List[Optional[np.ndarray]] = field(default_factory=list)
    idx16: List[Optional[np.ndarray]] = field(default_factory=list)
    codebooks: List[np.ndarray] = field(default_factory=list)   # float16 [2^b, 8]
    scales: Optional[np.ndarray] = None                          # float16 [N, nblk]
    stage_bits: Optional[List[int]] = None                       # per-stage widths (None: uniform)
    stage_scales: Optional[np.ndarray] = None                    # float32 [S] (None: all 1)
    sparse: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None  # CSR (rowptr, col, fp16 val)
    lowrank: Optional[Tuple[np.ndarray, np.ndarray]] = None  # fp16 U [N, r], V [r, K]

    @property
    def n_groups(self) -> int:
        return self.n_out * (self.k_in // 8)

    @property
    def widths(self) -> List[int]:
        return list(self.stage_bits) if self.stage_bits is not None else [self.idx_bits] * self.n_stages


# name -> (shapes, stages, bits, codebook stds, scale_block (None = per row),
#          x dtype, batches, rht max block (None = no transform), seed index)
WORKLOADS: Dict[str, dict] = {
    "tiny": dict(shapes=[("w", 256, 512)], stages=1, bits=8, cb_sd=(0.02,), scale_block=None,
                 x_dtype="f32", batches=(1,), rht=None, seed=0),
    "smollm": dict(shapes=[("q", 576, 576), ("k", 576, 576), ("v", 576, 576), ("o", 576, 576),
                           ("gate", 1536, 576), ("up", 1536, 576), ("down", 576, 1536)],
                   stages=1, bits=12, cb_sd=(0.02,), scale_block=128, x_dtype="bf16", batches=(1,),
                   rht=None, seed=1),
    "llama8b": dict(shapes=[("qo", 4096, 4096), ("gate_up", 14336, 4096), ("down", 4096, 14336)],
                    stages=2, bits=12, cb_sd=(0.02, 0.006), scale_block=128, x_dtype="bf16",
                    batches=(1, 16), rht=None, seed=2),
    "mlp70b": dict(shapes=[("gate_up", 28672, 8192), ("down", 8192, 28672)], stages=1, bits=16,
                   cb_sd=(0.02,), scale_block=None, x_dtype="bf16", batches=(1,), rht=8192, seed=3),
    "prefill": dict(shapes=[("qo", 4096, 4096), ("gate_up", 14336, 4096)], stages=2, bits=12,
                    cb_sd=(0.02, 0.006), scale_block=128, x_dtype="bf16", batches=(2048,), rht=None,
                    seed=4),
    "smollm_rvq124": dict(shapes=[("q", 576, 576), ("k", 576, 576), ("v", 576, 576), ("o", 576, 576),
                                  ("gate", 1536, 576), ("up", 1536, 576), ("down", 576, 1536)],
                          stages=2, bits=(12, 4), cb_sd=(0.02, 0.006), scale_block=128, x_dtype="bf16",
                          batches=(1,), rht=None, seed=5),
    "llama8b_rvq124": dict(shapes=[("qo", 4096, 4096), ("gate_up", 14336, 4096), ("down", 4096, 14336)],
                           stages=2, bits=(12, 4), cb_sd=(0.02, 0.006), scale_block=128, x_dtype="bf16",
                           batches=(1, 16), rht=None, seed=6),
    "llama8b_sparse": dict(shapes=[("qo", 4096, 4096), ("gate_up", 14336, 4096), ("down", 4096, 14336)],
                           stages=2, bits=12, cb_sd=(0.02, 0.006), scale_block=128, x_dtype="bf16",
                           batches=(1, 16), rht=None, seed=8, sparse=0.005),
    "llama8b_lowrank": dict(shapes=[("qo", 4096, 4096), ("gate_up", 14336, 4096), ("down", 4096, 14336)],
                            stages=2, bits=12, cb_sd=(0.02, 0.006), scale_block=128, x_dtype="bf16",
                            batches=(1, 16), rht=None, seed=9, lowrank=32),
    "mlp70b_e8p3": dict(shapes=[("gate_up", 28672, 8192), ("down", 8192, 28672)], stages=2, bits=(16, 8),
                        cb_sd=(0.02, 0.02), scale_block=None, x_dtype="bf16", batches=(1,), rht=8192, seed=7,
                        stage_scales=(0.2, 0.4)),
    "mlp70b_e8p4": dict(shapes=[("gate_up", 28672, 8192), ("down", 8192, 28672)], stages=2, bits=(16, 16),
                        cb_sd=(0.02, 0.02), scale_block=None, x_dtype="bf16", batches=(1,), rht=8192, seed=10,
                        stage_scales=(0.2, 0.4)),
}


def _rng(seed_seq: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq))


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns bits."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_weight(name: str, n_out: int, k_in: int, n_stages: int, idx_bits,
                cb_sd: Tuple[float, ...], scale_block: Optional[int],
                seed_seq: np.random.SeedSequence,
                stage_scale_range: Optional[Tuple[float, float]] = None,
                sparse_density: float = 0.0, lowrank_rank: int = 0) -> SynthWeight:
    """Draw one compressed weight.  ``idx_bits`` is one width for every stage
    or a list of per-stage widths (4, 8, 12, 16).  Draw order per stage:
    codebook, indices; then the scales; then, if ``stage_scale_range`` is
    given, the residual scales of stages 1.. (uniform on the range, rounded
    to float32; stage 0's is 1); then, if ``sparse_density`` > 0, a sparse
    correction: per row round(density * K) distinct columns (ascending),
    values N(0, 0.05) rounded to fp16; then, if ``lowrank_rank`` r > 0, the
    low-rank factors U [N, r] ~ N(0, 0.05) and V [r, K] ~ N(0, 0.05 / sqrt(r)),
    rounded to fp16 (entries of U V about 0.0025, an eighth of a weight)."""
    if k_in % 8:
        raise ValueError("k_in must be a multiple of 8")
    widths = [int(idx_bits)] * n_stages if np.isscalar(idx_bits) else [int(b) for b in idx_bits]
    if len(widths) != n_stages:
        raise ValueError("one index width per stage")
    bs = k_in if scale_block is None else scale_block
    rng = _rng(seed_seq)
    w = SynthWeight(name, n_out, k_in, n_stages, widths[0], bs,
                    stage_bits=None if len(set(widths)) == 1 else widths)
    ng = w.n_groups
    for t, b in enumerate(widths):
        cb = (rng.standard_normal((1 << b, 8)) * cb_sd[t]).astype(np.float16)
        w.codebooks.append(cb)
        if b == 16:
            w.idx16.append(rng.integers(0, 1 << 16, ng, dtype=np.uint16))
            w.lo.append(None)
            w.hi.append(None)
        elif b == 4:
            hi = rng.integers(0, 256, (ng + 1) // 2, dtype=np.uint8)
            if ng % 2:
                hi[-1] &= 0x0F
            w.idx16.append(None)
            w.lo.append(None)
            w.hi.append(hi)
        else:
            w.idx16.append(None)
            w.lo.append(rng.integers(0, 256, ng, dtype=np.uint8))
            if b == 12:
                hi = rng.integers(0, 256, (ng + 1) // 2, dtype=np.uint8)
                if ng % 2:
                    hi[-1] &= 0x0F
                w.hi.append(hi)
            else:
                w.hi.append(None)
    nblk = -(-k_in // bs)
    w.scales = rng.uniform(0.5, 1.5, (n_out, nblk)).astype(np.float16)
    if stage_scale_range is not None:
        lo_r, hi_r = stage_scale_range
        rs = np.ones(n_stages, np.float32)
        rs[1:] = rng.uniform(lo_r, hi_r, n_stages - 1).astype(np.float32)
        w.stage_scales = rs
    if sparse_density > 0:
        per = max(1, int(round(sparse_density * k_in)))
        cols = np.sort(np.argsort(rng.random((n_out, k_in)), axis=1)[:, :per], axis=1) if n_out * k_in <= (1 << 24) \
            else np.stack([np.sort(rng.choice(k_in, per, replace=False)) for _ in range(n_out)])
        rowptr = np.arange(n_out + 1, dtype=np.int64) * per
        val = (rng.standard_normal(n_out * per) * 0.05).astype(np.float16)
        w.sparse = (rowptr, cols.reshape(-1).astype(np.int64), val)
    if lowrank_rank > 0:
        u = (rng.standard_normal((n_out, lowrank_rank)) * 0.05).astype(np.float16)
        v = (rng.standard_normal((lowrank_rank, k_in)) * (0.05 / np.sqrt(lowrank_rank))).astype(np.float16)
        w.lowrank = (u, v)
    return w


def make_x(batch: int, k_in: int, dtype: str, seed_seq: np.random.SeedSequence):
    """Standard-normal activations.  Returns (stored array, float64 values):
    bf16 -> (uint16 bits, values); f32 -> (float32, values)."""
    v = _rng(seed_seq).standard_normal((batch, k_in)).astype(np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(v)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "f32":
        return v, v.astype(np.float64)
    raise ValueError(dtype)


def make_signs(n: int, seed_seq: np.random.SeedSequence) -> np.ndarray:
    """Random +/-1 signs (int8) for the input Hadamard transform."""
    return (_rng(seed_seq).integers(0, 2, n) * 2 - 1).astype(np.int8)


def workload_weights(workload: str, only: Optional[List[str]] = None, base_seed: int = 1000):
    """All weights of a workload, each from its own child seed stream of
    SeedSequence(base_seed + index).  Returns (weights, activation_seed_seq)."""
    cfg = WORKLOADS[workload]
    root = np.random.SeedSequence(base_seed + cfg["seed"])
    kids = root.spawn(len(cfg["shapes"]) + 1)
    out = []
    for (nm, n, k), ss in zip(cfg["shapes"], kids[:-1]):
        if only is not None and nm not in only:
            continue
        out.append(make_weight(nm, n, k, cfg["stages"], cfg["bits"], cfg["cb_sd"], cfg["scale_block"], ss,
                               cfg.get("stage_scales"), cfg.get("sparse", 0.0), cfg.get("lowrank", 0)))
    return out, kids[-1]


def random_weight(n_out, k_in, n_stages, idx_bits, scale_block, seed, cb_sd=None, stage_scale_range=None,
                  sparse_density=0.0, lowrank_rank=0):
    """A weight of any shape/format for ragged and edge-case tests."""
    sd = cb_sd or tuple(0.02 * (0.3 ** t) for t in range(n_stages))
    return make_weight(f"r{n_out}x{k_in}", n_out, k_in, n_stages, idx_bits, sd, scale_block,
                       np.random.SeedSequence(seed), stage_scale_range, sparse_density, lowrank_rank)
