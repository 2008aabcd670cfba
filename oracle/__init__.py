"""CPU oracle for the compressed-index matmul -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy statements of what the hot path computes, written
from the two source pages:

* orka README (github.com/orkait/orka.py), section "How it works": each group of
  8 weights is replaced by an index into a per-tensor codebook, the indices
  are stored as 12-bit bit-planes (a low-byte plane plus a plane of packed
  high nibbles), and a group is decoded as the scale times the sum of the
  codebook entries it indexes (one entry per residual stage).
* GLQ PyPI page ("GLQ -- fit larger LLMs on smaller GPUs"), sections
  "Inference kernels" (the product Y = X dequant(W)^T taken without forming W;
  each output row walks its K/8 codebook groups), "How it works" (randomized
  Hadamard transform = random sign flips followed by a fast Walsh-Hadamard
  transform; block-diagonal for large layers) and "Bit widths" (non-power-of-2
  sizes use a block-diagonal FHT built from power-of-2 blocks; 16-bit indices
  into a 65,536-entry codebook; higher rates stack 8- or 16-bit residual
  stages on a 16-bit primary), and the two-stage call of "Inference kernels",
  which passes an inverse residual scale.
* orka README, quick start: the ``rvq-12-4`` quant mode (a 12-bit primary
  stage and a 4-bit residual stage, about 2 bits per weight); "How it works"
  and the ``correct`` command of its CLI: the decode may add a sparse
  correction, and ``correct`` adds a low-rank or sparse correction.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library and
imports nothing from it.

Every function below is pinned by ``tests/test_oracle_*.py`` against closed
forms, hand-computed fixtures (``tests/golden/``), exact rational brute force,
or an independent library routine (``scipy.linalg.hadamard``, Python's
``struct`` half-float packing).  Where the pages leave a step open, the
reading taken is stated in the docstring.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Union

import numpy as np

__all__ = [
    "GROUP",
    "unpack_indices",
    "pack_indices",
    "n_scale_blocks",
    "dequant_exact",
    "dequant_fp16",
    "sparse_dense",
    "lowrank_dense",
    "lowrank_bound",
    "matmul_ref",
    "within_tolerance",
    "rht_blocks",
    "fwht",
    "rht_ref",
    "compressed_bytes",
    "bits_per_weight",
    "MATMUL_RTOL",
    "MATMUL_ATOL",
]

#: Weights per codebook group (orka README, "How it works": groups of 8).
GROUP = 8

#: Matmul acceptance bound |y - y_ref| <= MATMUL_RTOL * sum|w x| + MATMUL_ATOL.
MATMUL_RTOL = 2e-3
MATMUL_ATOL = 1e-6


# --------------------------------------------------------------------------
# c-1  index storage: bit-plane unpack
# --------------------------------------------------------------------------

def unpack_indices(bits: int, n_groups: int, lo=None, hi=None, idx16=None) -> np.ndarray:
    """Recover the codebook index of each of ``n_groups`` groups (flat order).

    orka README, "How it works": 12-bit indices are stored as bit-planes, a
    low-byte plane plus packed high bits.  Readings taken (the page is silent):

    * two planes, not twelve one-bit planes: ``lo`` holds bits 0..7 of every
      index, one byte per group; ``hi`` holds bits 8..11, two groups per byte;
    * group ``f`` uses the low nibble of ``hi[f // 2]`` when ``f`` is even and
      the high nibble when ``f`` is odd;
    * an 8-bit index is the ``lo`` plane alone;
    * a 16-bit index (GLQ "How it works": one 16-bit index per 8 weights into
      a 65,536-entry codebook) is a little-endian uint16 array ``idx16``;
    * a 4-bit index (the residual stage of orka's ``rvq-12-4`` mode) is one
      nibble plane ``hi``, packed exactly like the 12-bit high plane, so a
      12-bit index is an 8-bit ``lo`` plane plus a 4-bit plane shifted up by 8.

    Groups are numbered row-major: group ``g`` of output row ``r`` is
    ``f = r * (K // 8) + g``.
    """
    out = np.empty(n_groups, dtype=np.int64)
    if bits == 4:
        hib = np.asarray(hi, dtype=np.uint8)[np.arange(n_groups) // 2].astype(np.int64)
        out[:] = np.where(np.arange(n_groups) % 2 == 0, hib & 0xF, (hib >> 4) & 0xF)
    elif bits == 8:
        out[:] = np.asarray(lo, dtype=np.uint8)[:n_groups].astype(np.int64)
    elif bits == 12:
        lo = np.asarray(lo, dtype=np.uint8)
        hi = np.asarray(hi, dtype=np.uint8)
        f = np.arange(n_groups)
        low = lo[:n_groups].astype(np.int64)
        hib = hi[f // 2].astype(np.int64)
        nib = np.where(f % 2 == 0, hib & 0xF, (hib >> 4) & 0xF)
        out[:] = low + nib * 256
    elif bits == 16:
        arr = np.asarray(idx16)
        if arr.dtype != np.uint16:
            raise TypeError("16-bit indices must be a uint16 array")
        out[:] = arr[:n_groups].astype(np.int64)
    else:
        raise ValueError(f"unsupported index width {bits}")
    return out


def pack_indices(idx: Sequence[int], bits: int):
    """Inverse of :func:`unpack_indices` (used to build structured test inputs).

    Returns ``(lo, hi)`` for 8/12-bit (``hi`` is None for 8-bit),
    ``(None, hi)`` for 4-bit, or ``(idx16, None)`` for 16-bit.  For an odd
    number of 4/12-bit groups the unused high nibble of the last ``hi`` byte
    is zero.
    """
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= (1 << bits)):
        raise ValueError("index out of range for the width")
    if bits == 8:
        return idx.astype(np.uint8), None
    if bits == 16:
        return idx.astype(np.uint16), None
    if bits not in (4, 12):
        raise ValueError(f"unsupported index width {bits}")
    n = idx.size
    nib = np.zeros(2 * ((n + 1) // 2), dtype=np.int64)
    nib[:n] = idx // 256 if bits == 12 else idx
    hi = (nib[0::2] + 16 * nib[1::2]).astype(np.uint8)   # even group -> low nibble
    if bits == 4:
        return None, hi
    return (idx % 256).astype(np.uint8), hi


# --------------------------------------------------------------------------
# c-2  dequant
# --------------------------------------------------------------------------

def n_scale_blocks(k_in: int, scale_block: int) -> int:
    """Scales per row: one per ``scale_block`` input columns, the last block
    possibly short (ceil reading; e.g. K=576 with 128-column blocks gives 5)."""
    return -(-k_in // scale_block)


def dequant_exact(n_out: int, k_in: int, indices: Sequence[np.ndarray],
                  codebooks: Sequence[np.ndarray], scales: np.ndarray,
                  scale_block: int, stage_scales: Optional[Sequence[float]] = None,
                  sparse=None, lowrank=None) -> np.ndarray:
    """Dequantized weight, float64, shape ``[n_out, k_in]``.

    orka README, "How it works": a group decodes to the scale times the sum of
    its codebook entries; with residual stages t = 0..S-1 (orka's RVQ, GLQ
    "Bit widths" residual stages) this is

        w[r, 8g + j] = s[r, (8g) // scale_block] * sum_t cb_t[idx_t[r, g], j].

    Readings: the scale multiplies the stage sum; one block scale is shared by
    all stages.  All values are fp16, so the sum of at most four of them and
    its product with an fp16 scale are exact in float64 -- the result does not
    depend on summation order (the sign of an exact zero included: it is -0
    only when every term is -0).

    ``stage_scales`` (optional, one float32 per stage) is the residual scale
    of GLQ's two-stage call ("Inference kernels": an inverse residual scale)
    and of its stacked trellis stages (a residual scale fitted per layer):

        w[r, 8g + j] = s[r, blk] * sum_t r_t * cb_t[idx_t[r, g], j].

    Readings: one scalar per stage per tensor, multiplying that stage's
    codebook entry, any stage (the primary included) may carry one, and
    omitting them means r_t = 1.  With them the value is no longer exact in
    float64 in general, so it is defined by this evaluation order: each
    product r_t * c_t (exact in float64: 24 + 11 significant bits), summed in
    stage order starting from stage 0's product, each addition rounded to
    float64, then one float64 multiplication by the block scale.  With every
    r_t = 1 this is the exact value above, bit for bit.

    ``sparse`` (CSR ``(rowptr, col, val)``, fp16 values) is the sparse
    correction of orka's decode ("How it works"): each entry is added to its
    weight after the block scale, a row's entries in storage order.

    ``lowrank`` (``(U, V)``: fp16 ``U [n_out, r]`` and ``V [r, k_in]``) is
    the low-rank correction of orka's ``correct`` command (CLI), whose form
    the pages do not give.  Reading: the correction is the product U V added
    to the decoded weight (after the sparse entries), w += sum_j U[:, j]
    V[j, :], each product exact in float64 (11 + 11 significant bits) and the
    rank-one terms added in order j = 0, 1, ..., each addition rounded to
    float64.
    """
    if k_in % GROUP:
        raise ValueError("k_in must be a multiple of 8")
    g_per_row = k_in // GROUP
    s = np.asarray(scales, dtype=np.float16).astype(np.float64).reshape(n_out, -1)
    if stage_scales is not None:
        rs = np.asarray(stage_scales, dtype=np.float32).astype(np.float64)
        if rs.size < len(codebooks):
            raise ValueError("one stage scale per stage")
        if not np.all(np.isfinite(rs)):
            raise ValueError("stage scales must be finite")
    acc = None
    for t, (idx, cb) in enumerate(zip(indices, codebooks)):
        cb64 = np.asarray(cb, dtype=np.float16).astype(np.float64).reshape(-1, GROUP)
        ix = np.asarray(idx, dtype=np.int64).reshape(n_out, g_per_row)
        term = cb64[ix]
        if stage_scales is not None:
            term = rs[t] * term          # exact: 24-bit times 11-bit significand
        # The sum starts from stage 0's term itself (not from +0), so a lone
        # -0.0 entry stays -0.0; an exact zero sum of mixed-sign terms is +0.
        acc = term if acc is None else acc + term
    if acc is None:
        raise ValueError("at least one stage is required")
    w = np.empty((n_out, k_in), dtype=np.float64)
    for g in range(g_per_row):
        blk = (GROUP * g) // scale_block
        w[:, GROUP * g:GROUP * (g + 1)] = s[:, blk:blk + 1] * acc[:, g, :]
    if sparse is not None:
        rowptr, col, val = _check_sparse(n_out, k_in, sparse)
        for r in range(n_out):
            for j in range(rowptr[r], rowptr[r + 1]):
                w[r, col[j]] = w[r, col[j]] + val[j]
    if lowrank is not None:
        u, v = _check_lowrank(n_out, k_in, lowrank)
        for j in range(u.shape[1]):
            w = w + np.outer(u[:, j], v[j])  # exact products, one rounding per addition
    return w


def _check_sparse(n_out: int, k_in: int, sparse):
    rowptr, col, val = sparse
    rowptr = np.asarray(rowptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    val = np.asarray(val, dtype=np.float16).astype(np.float64)
    if rowptr.shape != (n_out + 1,) or rowptr[0] != 0 or np.any(np.diff(rowptr) < 0):
        raise ValueError("rowptr must have n_out + 1 non-decreasing entries starting at 0")
    nnz = int(rowptr[-1])
    if col.size < nnz or val.size < nnz:
        raise ValueError("col and val need rowptr[n_out] entries")
    if nnz and (col[:nnz].min() < 0 or col[:nnz].max() >= k_in):
        raise ValueError("column out of range")
    return rowptr, col, val


def sparse_dense(n_out: int, k_in: int, sparse) -> np.ndarray:
    """The sparse correction alone as a dense float64 [n_out, k_in] matrix
    (entries of one row added in storage order)."""
    rowptr, col, val = _check_sparse(n_out, k_in, sparse)
    d = np.zeros((n_out, k_in), dtype=np.float64)
    for r in range(n_out):
        for j in range(rowptr[r], rowptr[r + 1]):
            d[r, col[j]] += val[j]
    return d


def _check_lowrank(n_out: int, k_in: int, lowrank):
    u, v = lowrank
    u = np.asarray(u, dtype=np.float16).astype(np.float64)
    v = np.asarray(v, dtype=np.float16).astype(np.float64)
    if u.ndim != 2 or v.ndim != 2 or u.shape[0] != n_out or v.shape[1] != k_in or u.shape[1] != v.shape[0]:
        raise ValueError("low-rank factors must be U [n_out, r] and V [r, k_in]")
    if u.shape[1] < 1:
        raise ValueError("rank must be at least 1")
    return u, v


def lowrank_dense(n_out: int, k_in: int, lowrank) -> np.ndarray:
    """The low-rank correction alone, U V, as a float64 [n_out, k_in]
    matrix (rank-one terms added in order j = 0, 1, ...)."""
    u, v = _check_lowrank(n_out, k_in, lowrank)
    d = np.zeros((n_out, k_in), dtype=np.float64)
    for j in range(u.shape[1]):
        d = d + np.outer(u[:, j], v[j])
    return d


def lowrank_bound(x: np.ndarray, lowrank) -> np.ndarray:
    """Error scale of applying the low-rank correction through its factors,
    y += (x V^T) U^T: ``bound[b, r] = sum_j |U[r, j]| sum_k |V[j, k] x[b, k]|``.

    Reading: the pages fix no precision for the correction; a product that
    never forms U V carries rounding relative to this scale, not to
    sum_k |(U V)[r, k] x[b, k]| (which cancellation in U V can make much
    smaller), so the matmul acceptance bound of a weight with a low-rank
    correction adds this term to :func:`matmul_ref`'s."""
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    u, v = lowrank
    u = np.asarray(u, dtype=np.float16).astype(np.float64)
    v = np.asarray(v, dtype=np.float16).astype(np.float64)
    return (np.abs(x64) @ np.abs(v).T) @ np.abs(u).T


def dequant_fp16(n_out, k_in, indices, codebooks, scales, scale_block,
                 stage_scales=None, sparse=None, lowrank=None) -> np.ndarray:
    """fp16 dequantized weight: the float64 value rounded once to nearest-even.

    Reading: the pages fix no rounding; the result is the float64 value of
    :func:`dequant_exact` (exact without stage scales, the stated evaluation
    order with them, plus the sparse and low-rank corrections if any)
    converted once to
    IEEE binary16 with
    round-to-nearest-even (numpy's float64 -> float16 cast rounds once; the
    tests check it against Python's own half-float packing).  Subnormals are
    kept, overflow gives +/-inf, a zero result keeps the sign IEEE gives it.
    """
    return dequant_exact(n_out, k_in, indices, codebooks, scales, scale_block,
                         stage_scales, sparse, lowrank).astype(np.float16)


# --------------------------------------------------------------------------
# c-3  matmul
# --------------------------------------------------------------------------

def matmul_ref(w64: np.ndarray, x: np.ndarray):
    """``Y = X dequant(W)^T`` (GLQ "Inference kernels") in float64.

    ``w64`` is the exact dequantized weight [N, K]; ``x`` is [B, K] (any float
    dtype; bf16/fp32 inputs are exact in float64).  Returns ``(y, bound)``
    where ``bound[b, r] = sum_k |w[r, k] * x[b, k]|`` is the scale of the
    acceptance test of :func:`within_tolerance`.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    w64 = np.asarray(w64, dtype=np.float64)
    y = x64 @ w64.T
    bound = np.abs(x64) @ np.abs(w64).T
    return y, bound


def within_tolerance(y, y_ref, bound, rtol: float = MATMUL_RTOL, atol: float = MATMUL_ATOL):
    """Per-output acceptance: |y - y_ref| <= rtol * bound + atol.  Returns a
    boolean array and the worst ratio |y - y_ref| / (rtol * bound + atol)."""
    y = np.asarray(y, dtype=np.float64)
    lim = rtol * np.asarray(bound, dtype=np.float64) + atol
    err = np.abs(y - np.asarray(y_ref, dtype=np.float64))
    ok = err <= lim
    worst = float(np.max(err / lim)) if err.size else 0.0
    return ok, worst


# --------------------------------------------------------------------------
# c-4  randomized Hadamard transform on the input
# --------------------------------------------------------------------------

def rht_blocks(n: int, max_block: int):
    """Block sizes of the block-diagonal transform for a length-``n`` vector.

    GLQ "Bit widths": a size that is not a power of two is split into
    power-of-two blocks (their example: 2688 = 2048 + 512 + 128).  Reading:
    greedy largest-first decomposition with every block capped at
    ``max_block`` (so 28672 with an 8192 cap is 8192, 8192, 8192, 4096).
    """
    if n <= 0:
        raise ValueError("n must be positive")
    if max_block <= 0 or (max_block & (max_block - 1)):
        raise ValueError("max_block must be a power of two")
    blocks = []
    rest = n
    while rest:
        b = min(max_block, 1 << (rest.bit_length() - 1))
        blocks.append(b)
        rest -= b
    return blocks


def fwht(v: np.ndarray) -> np.ndarray:
    """Orthonormal fast Walsh-Hadamard transform of a length-2^m vector,
    float64, natural (Sylvester) order: H_1 = [1], H_2n = [[H, H], [H, -H]],
    scaled by 1/sqrt(n) so that the transform is its own inverse."""
    a = np.array(v, dtype=np.float64, copy=True)
    n = a.size
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < n:
        a = a.reshape(-1, 2, h)
        top = a[:, 0, :] + a[:, 1, :]
        bot = a[:, 0, :] - a[:, 1, :]
        a = np.stack([top, bot], axis=1).reshape(n)
        h *= 2
    return a / math.sqrt(n)


def rht_ref(x: np.ndarray, signs: np.ndarray, max_block: int) -> np.ndarray:
    """Randomized Hadamard transform of each row of ``x`` [B, n], float64.

    GLQ "How it works": random sign flips, then a fast Walsh-Hadamard
    transform, block-diagonal for large sizes.  Readings: signs are applied
    first (x' = blockdiag(H_n1, ..., H_nm) (sigma * x)); each block uses the
    orthonormal Sylvester-order transform of :func:`fwht`; blocks follow
    :func:`rht_blocks`.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    sg = np.asarray(signs, dtype=np.float64)
    n = x64.shape[1]
    out = np.empty_like(x64)
    for b in range(x64.shape[0]):
        v = x64[b] * sg
        off = 0
        for blk in rht_blocks(n, max_block):
            out[b, off:off + blk] = fwht(v[off:off + blk])
            off += blk
    return out


def rht_inverse_ref(y: np.ndarray, signs: np.ndarray, max_block: int) -> np.ndarray:
    """Output-side transform of each row of ``y`` [B, n], float64: the inverse
    of :func:`rht_ref`.

    GLQ "How it works": the weights are rotated and the inverse transform runs
    inside the inference kernels; "Inference kernels" (the fused linear: input
    RHT, decode, scale, output RHT).  Reading: a weight stored rotated on its
    output side as W' = (H D) W, with D = diag(signs) and H the block-diagonal
    orthonormal Hadamard of :func:`rht_blocks`, gives W x = (H D)^T W' x, and
    (H D)^T = D H because H is symmetric: the blocks' Hadamard first, then the
    sign flips.
    """
    y64 = np.asarray(y, dtype=np.float64)
    if y64.ndim == 1:
        y64 = y64[None, :]
    sg = np.asarray(signs, dtype=np.float64)
    n = y64.shape[1]
    out = np.empty_like(y64)
    for b in range(y64.shape[0]):
        off = 0
        for blk in rht_blocks(n, max_block):
            out[b, off:off + blk] = fwht(y64[b, off:off + blk])
            off += blk
        out[b] *= sg
    return out


def rht_shards_ref(x: np.ndarray, shard_lens: Sequence[int], signs: np.ndarray, max_block: int,
                   inverse: bool = False) -> np.ndarray:
    """Shard-batched transform (GLQ "Inference kernels", shard-batched output
    RHT: the per-shard output transforms of a fused QKV or gate-up layer in
    one launch).  Each row of ``x`` [B, sum(shard_lens)] is cut into
    consecutive shards; every shard is transformed on its own, exactly as
    :func:`rht_ref` (or :func:`rht_inverse_ref` with ``inverse``) transforms
    a row of that length, with the signs of its own columns.  Reading: the
    block decomposition restarts at every shard boundary, because each shard
    is a separate linear whose rotation was chosen for its own size."""
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim == 1:
        x64 = x64[None, :]
    if sum(shard_lens) != x64.shape[1] or any(n <= 0 for n in shard_lens):
        raise ValueError("shard lengths must be positive and cover the row")
    fn = rht_inverse_ref if inverse else rht_ref
    out = np.empty_like(x64)
    off = 0
    for n in shard_lens:
        out[:, off:off + n] = fn(x64[:, off:off + n], signs[off:off + n], max_block)
        off += n
    return out


# --------------------------------------------------------------------------
# c-5  storage cost
# --------------------------------------------------------------------------

def _stage_widths(n_stages: int, bits) -> list:
    if isinstance(bits, (int, np.integer)):
        widths = [int(bits)] * n_stages
    else:
        widths = [int(b) for b in bits]
        if len(widths) != n_stages:
            raise ValueError("one index width per stage")
    for b in widths:
        if b not in (4, 8, 12, 16):
            raise ValueError(f"unsupported index width {b}")
    return widths


def compressed_bytes(n_out: int, k_in: int, n_stages: int, bits: Union[int, Sequence[int]],
                     scale_block: int, include_codebooks: bool = True, sparse_nnz: int = 0,
                     lowrank_rank: int = 0) -> int:
    """Bytes of the stored weight: index planes, fp16 scales and (optionally)
    the fp16 codebooks, each counted once.

    ``bits`` is one index width for every stage or a list of per-stage widths
    (GLQ "Bit widths": a 16-bit primary with 8- or 16-bit residual stages;
    orka's ``rvq-12-4``: 12 then 4).  Per stage: 16-bit = two bytes per
    group, 12-bit = one byte per group plus one byte per two groups (ceil),
    8-bit = one byte per group, 4-bit = one byte per two groups (ceil).
    A sparse correction of ``sparse_nnz`` entries adds its CSR arrays: int32
    row pointers (n_out + 1), int32 columns and fp16 values.  A low-rank
    correction of rank r adds its fp16 factors: 2 r (n_out + k_in) bytes.
    """
    groups = n_out * (k_in // GROUP)
    per_width = {4: (groups + 1) // 2, 8: groups, 12: groups + (groups + 1) // 2, 16: 2 * groups}
    widths = _stage_widths(n_stages, bits)
    total = sum(per_width[b] for b in widths) + 2 * n_out * n_scale_blocks(k_in, scale_block)
    if include_codebooks:
        total += sum((1 << b) * GROUP * 2 for b in widths)
    if sparse_nnz:
        total += 4 * (n_out + 1) + (4 + 2) * sparse_nnz
    if lowrank_rank:
        total += 2 * lowrank_rank * (n_out + k_in)
    return total


def bits_per_weight(n_out: int, k_in: int, n_stages: int, bits: Union[int, Sequence[int]],
                    scale_block: int, include_codebooks: bool = False) -> float:
    """Stored bits per weight: b/8 per stage for the indices (12 bits per 8
    weights is 1.5 per stage) plus 16 bits per scale block, plus optionally
    the codebooks spread over the tensor."""
    return 8.0 * compressed_bytes(n_out, k_in, n_stages, bits, scale_block,
                                  include_codebooks) / (n_out * k_in)
