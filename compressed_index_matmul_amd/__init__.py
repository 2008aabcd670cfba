"""Python binding of libvqmm, the gfx950 compressed-index matmul library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/vqmm.h``.  PyTorch supplies
device memory and the current stream.  There is no fallback: if the shared
library is missing or fails to load, every entry point raises.

Entry points (same names as the C ABI):

* :func:`vq_unpack_dequant` -- unpacked indices and/or the fp16 dense weight
* :func:`vq_gemv`           -- y = x dequant(W)^T for 1..16 tokens
* :func:`vq_gemm`           -- the same for many bf16 tokens on matrix cores
* :func:`rht_apply`         -- randomized Hadamard transform of activations
* :func:`vq_compressed_bytes`, :func:`vq_validate`, :func:`vq_version`
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "VQError", "VQWeight", "lib", "LIB_PATH", "vq_version", "vq_validate", "vq_compressed_bytes",
    "vq_unpack_dequant", "vq_gemv", "vq_gemm", "rht_apply", "vq_gemv_rht", "VQ_F32", "VQ_BF16", "VQ_STAGE_SCALES",
    "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvqmm.so")
VQ_F32, VQ_BF16 = 0, 1
MAX_STAGES = 4
EXPORTS = ("vq_version", "vq_status_string", "vq_validate", "vq_compressed_bytes",
           "vq_unpack_dequant", "vq_gemv", "vq_gemm", "rht_apply", "vq_gemv_rht")

_ptr4 = ctypes.c_void_p * MAX_STAGES
_int4 = ctypes.c_int32 * MAX_STAGES
_flt4 = ctypes.c_float * MAX_STAGES
VQ_STAGE_SCALES = 1


class VQWeightDesc(ctypes.Structure):
    """Mirror of ``struct vq_weight``."""
    _fields_ = [
        ("n_out", ctypes.c_int32),
        ("k_in", ctypes.c_int32),
        ("n_stages", ctypes.c_int32),
        ("idx_bits", ctypes.c_int32),
        ("scale_block", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("idx_lo", _ptr4),
        ("idx_hi", _ptr4),
        ("idx16", _ptr4),
        ("codebook", _ptr4),
        ("scales", ctypes.c_void_p),
        ("stage_bits", _int4),
        ("stage_scale", _flt4),
        ("sp_nnz", ctypes.c_int32),
        ("sp_reserved", ctypes.c_int32),
        ("sp_rowptr", ctypes.c_void_p),
        ("sp_col", ctypes.c_void_p),
        ("sp_val", ctypes.c_void_p),
    ]


class VQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} (status {status})")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_index_matmul_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(VQWeightDesc)
        L.vq_version.argtypes, L.vq_version.restype = [], ctypes.c_int
        L.vq_status_string.argtypes, L.vq_status_string.restype = [ctypes.c_int], ctypes.c_char_p
        L.vq_validate.argtypes, L.vq_validate.restype = [D], ctypes.c_int
        L.vq_compressed_bytes.argtypes, L.vq_compressed_bytes.restype = [D], ctypes.c_int64
        L.vq_unpack_dequant.argtypes, L.vq_unpack_dequant.restype = [D, P, P, P], ctypes.c_int
        L.vq_gemv.argtypes = [D, P, ctypes.c_int32, ctypes.c_int32, P, P]
        L.vq_gemv.restype = ctypes.c_int
        L.vq_gemm.argtypes, L.vq_gemm.restype = [D, P, ctypes.c_int32, P, P], ctypes.c_int
        L.rht_apply.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P, P]
        L.rht_apply.restype = ctypes.c_int
        L.vq_gemv_rht.argtypes = [D, P, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P, P]
        L.vq_gemv_rht.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _status_string(st: int) -> str:
    try:
        return lib().vq_status_string(st).decode()
    except Exception:  # pragma: no cover
        return "unknown"


def _check(st: int, what: str) -> None:
    if st != 0:
        raise VQError(st, what)


def vq_version() -> int:
    return lib().vq_version()


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _as_device(a, device, dtype=None):
    import torch
    if isinstance(a, torch.Tensor):
        t = a
    else:
        arr = np.ascontiguousarray(a)
        if arr.dtype == np.uint16:
            arr = arr.view(np.int16)
        t = torch.from_numpy(arr)
    if dtype is not None and t.dtype != dtype:
        t = t.view(dtype) if t.element_size() == torch.empty((), dtype=dtype).element_size() else t.to(dtype)
    return t.to(device).contiguous()


class VQWeight:
    """A compressed weight resident in device memory plus its descriptor.

    The tensors are kept alive by this object; the descriptor holds their
    raw device addresses.  ``stage_bits`` (optional) gives each stage its own
    index width (4, 8, 12 or 16); ``stage_scales`` (optional) one float
    residual scale per stage; ``sparse`` (optional) a CSR correction
    ``(rowptr, col, val)`` added to the decoded weight.
    """

    def __init__(self, n_out: int, k_in: int, n_stages: int, idx_bits: int, scale_block: int,
                 codebooks: Sequence, scales, lo: Sequence = (), hi: Sequence = (),
                 idx16: Sequence = (), device="cuda", stage_bits: Optional[Sequence[int]] = None,
                 stage_scales: Optional[Sequence[float]] = None, sparse=None):
        import torch
        self.n_out, self.k_in, self.n_stages, self.idx_bits = n_out, k_in, n_stages, idx_bits
        self.scale_block = scale_block
        self.stage_bits = None if stage_bits is None else [int(b) for b in stage_bits]
        self.stage_scales = None if stage_scales is None else [float(np.float32(r)) for r in stage_scales]
        self.device = torch.device(device)
        self.codebooks = [_as_device(c, self.device, torch.float16) for c in codebooks]
        self.scales = _as_device(scales, self.device, torch.float16)
        self.lo = [None if v is None else _as_device(v, self.device, torch.uint8) for v in lo]
        self.hi = [None if v is None else _as_device(v, self.device, torch.uint8) for v in hi]
        self.idx16 = [None if v is None else _as_device(v, self.device, torch.int16) for v in idx16]
        self.sparse = None
        if sparse is not None:
            rp, cl, vl = sparse
            self.sparse = (_as_device(np.asarray(rp, np.int32), self.device, torch.int32),
                           _as_device(np.asarray(cl, np.int32), self.device, torch.int32),
                           _as_device(np.asarray(vl, np.float16), self.device, torch.float16))
        self.desc = VQWeightDesc()
        self._fill_desc()

    def _fill_desc(self):
        d = self.desc
        d.n_out, d.k_in, d.n_stages, d.idx_bits = self.n_out, self.k_in, self.n_stages, self.idx_bits
        d.scale_block = self.scale_block
        d.flags = 0 if self.stage_scales is None else VQ_STAGE_SCALES
        for t in range(MAX_STAGES):
            d.stage_bits[t] = self.stage_bits[t] if self.stage_bits is not None and t < len(self.stage_bits) else 0
            d.stage_scale[t] = (self.stage_scales[t] if self.stage_scales is not None and t < len(self.stage_scales)
                                else 1.0)
        for t in range(MAX_STAGES):
            d.idx_lo[t] = self.lo[t].data_ptr() if t < len(self.lo) and self.lo[t] is not None else None
            d.idx_hi[t] = self.hi[t].data_ptr() if t < len(self.hi) and self.hi[t] is not None else None
            d.idx16[t] = self.idx16[t].data_ptr() if t < len(self.idx16) and self.idx16[t] is not None else None
            d.codebook[t] = self.codebooks[t].data_ptr() if t < len(self.codebooks) else None
        d.scales = self.scales.data_ptr()
        nnz = 0 if self.sparse is None else int(self.sparse[1].numel())
        d.sp_nnz, d.sp_reserved = nnz, 0
        d.sp_rowptr = self.sparse[0].data_ptr() if nnz else None
        d.sp_col = self.sparse[1].data_ptr() if nnz else None
        d.sp_val = self.sparse[2].data_ptr() if nnz else None

    def clone(self) -> "VQWeight":
        """Another copy of the same weight at distinct device addresses."""
        w = VQWeight.__new__(VQWeight)
        w.__dict__.update({k: v for k, v in self.__dict__.items() if k not in ("desc",)})
        w.codebooks = [c.clone() for c in self.codebooks]
        w.scales = self.scales.clone()
        w.lo = [None if v is None else v.clone() for v in self.lo]
        w.hi = [None if v is None else v.clone() for v in self.hi]
        w.idx16 = [None if v is None else v.clone() for v in self.idx16]
        w.sparse = None if self.sparse is None else tuple(t.clone() for t in self.sparse)
        w.desc = VQWeightDesc()
        w._fill_desc()
        return w

    def nbytes_device(self) -> int:
        ts = [*self.codebooks, self.scales, *[v for v in self.lo + self.hi + self.idx16 if v is not None],
              *(self.sparse or ())]
        return sum(t.numel() * t.element_size() for t in ts)

    def ref(self):
        return ctypes.byref(self.desc)


def vq_validate(w: VQWeight) -> int:
    return lib().vq_validate(w.ref())


def vq_compressed_bytes(w: VQWeight) -> int:
    v = lib().vq_compressed_bytes(w.ref())
    if v < 0:
        raise VQError(int(v), "vq_compressed_bytes")
    return int(v)


def _xtype(x) -> int:
    import torch
    if x.dtype == torch.float32:
        return VQ_F32
    if x.dtype == torch.bfloat16:
        return VQ_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def vq_unpack_dequant(w: VQWeight, want_idx: bool = True, want_w: bool = True, stream=None):
    """Returns (idx [S, N, K/8] int32-viewable uint16 as torch.int16, w fp16 [N, K])."""
    import torch
    idx = torch.empty((w.n_stages, w.n_out, w.k_in // 8), dtype=torch.int16, device=w.device) if want_idx else None
    wt = torch.empty((w.n_out, w.k_in), dtype=torch.float16, device=w.device) if want_w else None
    _check(lib().vq_unpack_dequant(w.ref(), idx.data_ptr() if idx is not None else None,
                                   wt.data_ptr() if wt is not None else None, _stream_handle(stream)),
           "vq_unpack_dequant")
    return idx, wt


def vq_gemv(w: VQWeight, x, y=None, stream=None):
    """x: [B, K] (B <= 16) float32 or bfloat16 on the device -> y float32 [B, N]."""
    import torch
    if x.dim() == 1:
        x = x.unsqueeze(0)
    x = x.contiguous()
    b = x.shape[0]
    if y is None:
        y = torch.empty((b, w.n_out), dtype=torch.float32, device=x.device)
    _check(lib().vq_gemv(w.ref(), x.data_ptr(), _xtype(x), b, y.data_ptr(), _stream_handle(stream)), "vq_gemv")
    return y


def vq_gemm(w: VQWeight, x, y=None, stream=None):
    """x: bfloat16 [M, K] on the device -> y float32 [M, N]."""
    import torch
    if x.dtype != torch.bfloat16:
        raise TypeError("vq_gemm takes bfloat16 activations")
    x = x.contiguous()
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, w.n_out), dtype=torch.float32, device=x.device)
    _check(lib().vq_gemm(w.ref(), x.data_ptr(), m, y.data_ptr(), _stream_handle(stream)), "vq_gemm")
    return y


def rht_apply(x, signs, max_block: int, out=None, stream=None):
    """x: [B, n] float32/bfloat16, signs int8 [n] on the device -> float32 [B, n]."""
    import torch
    if x.dim() == 1:
        x = x.unsqueeze(0)
    x = x.contiguous()
    b, n = x.shape
    if out is None:
        out = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _check(lib().rht_apply(x.data_ptr(), _xtype(x), b, n, signs.data_ptr(), max_block, out.data_ptr(),
                           _stream_handle(stream)), "rht_apply")
    return out


def vq_gemv_rht(w: VQWeight, x, signs, max_block: int, y=None, stream=None):
    """y = dequant(W) . RHT(x) with the transform inside the decode kernel:
    x [B, K] (B <= 16) float32/bfloat16, signs int8 [K] on the device -> y
    float32 [B, N].  Raises VQError (VQ_ERR_UNSUPPORTED) for weights the
    16-bit decode kernel does not take."""
    import torch
    if x.dim() == 1:
        x = x.unsqueeze(0)
    x = x.contiguous()
    b = x.shape[0]
    if y is None:
        y = torch.empty((b, w.n_out), dtype=torch.float32, device=x.device)
    _check(lib().vq_gemv_rht(w.ref(), x.data_ptr(), _xtype(x), b, signs.data_ptr(), max_block, y.data_ptr(),
                             _stream_handle(stream)), "vq_gemv_rht")
    return y
