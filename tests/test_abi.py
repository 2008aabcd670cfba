"""The C-ABI library loads without a GPU, exports every symbol the header
declares, and rejects every invalid argument on the host before touching the
device (no compute calls here)."""
import ctypes
import os
import re

import pytest

import oracle
import vqsynth
from vqtest import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "vqmm.h")

VQ_OK, VQ_ERR_NULL, VQ_ERR_SHAPE, VQ_ERR_DTYPE, VQ_ERR_UNSUPPORTED, VQ_ERR_ALIGN, VQ_ERR_HIP, VQ_ERR_VALUE, \
    VQ_ERR_WORKSPACE = 0, -1, -2, -3, -4, -5, -6, -7, -8
FAKE = 0x10000  # 16-byte aligned stand-in address, never dereferenced by validation


@pytest.fixture(scope="module")
def L():
    ensure_built()
    import compressed_index_matmul_amd as vq
    return vq.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_resolves_every_symbol():
    """Load with immediate binding: an undefined symbol (for example a kernel
    launch stub the compiler dropped) fails here rather than on the GPU."""
    ensure_built()
    from compressed_index_matmul_amd import LIB_PATH
    ctypes.CDLL(LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("vq_unpack_dequant", "vq_gemv", "vq_gemm", "vq_gemm_workspace_size", "rht_apply", "vq_version",
                 "vq_status_string", "vq_validate", "vq_compressed_bytes"):
        assert name in fns


def test_exports_every_declared_symbol(L):
    import compressed_index_matmul_amd as vq
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) == set(vq.EXPORTS)


def test_version_matches_header(L):
    m = re.search(r"#define VQMM_VERSION (\d+)", open(HEADER).read())
    assert L.vq_version() == int(m.group(1))


def test_status_strings(L):
    for st in (VQ_OK, VQ_ERR_NULL, VQ_ERR_SHAPE, VQ_ERR_DTYPE, VQ_ERR_UNSUPPORTED, VQ_ERR_ALIGN, VQ_ERR_HIP,
               VQ_ERR_VALUE, VQ_ERR_WORKSPACE):
        s = L.vq_status_string(st).decode()
        assert s and s != "unknown status"
    assert L.vq_status_string(12345).decode() == "unknown status"


def fake_desc(n=64, k=64, stages=1, bits=12, bs=32, widths=None, stage_scales=None):
    """A descriptor of stand-in addresses; ``widths`` gives per-stage widths
    (stage_bits), ``stage_scales`` sets VQ_STAGE_SCALES."""
    from compressed_index_matmul_amd import VQWeightDesc, VQ_STAGE_SCALES
    d = VQWeightDesc()
    d.n_out, d.k_in, d.n_stages, d.idx_bits, d.scale_block = n, k, stages, bits, bs
    ws = widths or [bits] * stages
    for t in range(stages):
        d.codebook[t] = FAKE
        b = ws[t]
        if widths is not None:
            d.stage_bits[t] = b
        if b == 16:
            d.idx16[t] = FAKE
        if b in (8, 12):
            d.idx_lo[t] = FAKE
        if b in (4, 12):
            d.idx_hi[t] = FAKE
    if stage_scales is not None:
        d.flags = VQ_STAGE_SCALES
        for t, r in enumerate(stage_scales):
            d.stage_scale[t] = r
    d.scales = FAKE
    return d


def test_valid_descriptors(L):
    for bits in (8, 12, 16):
        for st in (1, 2, 3, 4):
            d = fake_desc(stages=st, bits=bits)
            assert L.vq_validate(ctypes.byref(d)) == VQ_OK


@pytest.mark.parametrize("mutate,code", [
    (lambda d: setattr(d, "n_out", 0), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "k_in", 12), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "k_in", 0), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "n_stages", 0), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "n_stages", 5), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "idx_bits", 10), VQ_ERR_UNSUPPORTED),
    (lambda d: setattr(d, "scale_block", 4), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "scale_block", 20), VQ_ERR_SHAPE),
    (lambda d: d.codebook.__setitem__(0, None), VQ_ERR_NULL),
    (lambda d: d.idx_hi.__setitem__(0, None), VQ_ERR_NULL),
    (lambda d: d.idx_lo.__setitem__(0, None), VQ_ERR_NULL),
    (lambda d: setattr(d, "scales", None), VQ_ERR_NULL),
    (lambda d: d.codebook.__setitem__(0, FAKE + 8), VQ_ERR_ALIGN),
    (lambda d: d.idx_lo.__setitem__(0, FAKE + 4), VQ_ERR_ALIGN),
    (lambda d: setattr(d, "scales", FAKE + 2), VQ_ERR_ALIGN),
    (lambda d: (setattr(d, "n_out", 1 << 20), setattr(d, "k_in", 1 << 12)), VQ_ERR_SHAPE),
])
def test_invalid_descriptor(L, mutate, code):
    d = fake_desc()
    mutate(d)
    assert L.vq_validate(ctypes.byref(d)) == code
    # every compute entry point returns the same code, before any HIP call
    assert L.vq_gemv(ctypes.byref(d), FAKE, 1, 1, FAKE, None) == code
    assert L.vq_gemm(ctypes.byref(d), FAKE, 64, FAKE, None, 0, None) == code
    assert L.vq_unpack_dequant(ctypes.byref(d), FAKE, FAKE, None) == code
    assert L.vq_compressed_bytes(ctypes.byref(d)) == code


def test_null_descriptor(L):
    assert L.vq_validate(None) == VQ_ERR_NULL
    assert L.vq_gemv(None, FAKE, 1, 1, FAKE, None) == VQ_ERR_NULL


def test_gemv_argument_checks(L):
    d = ctypes.byref(fake_desc())
    assert L.vq_gemv(d, None, 1, 1, FAKE, None) == VQ_ERR_NULL
    assert L.vq_gemv(d, FAKE, 1, 1, None, None) == VQ_ERR_NULL
    assert L.vq_gemv(d, FAKE, 7, 1, FAKE, None) == VQ_ERR_DTYPE
    assert L.vq_gemv(d, FAKE, 1, 0, FAKE, None) == VQ_ERR_UNSUPPORTED
    assert L.vq_gemv(d, FAKE, 1, 17, FAKE, None) == VQ_ERR_UNSUPPORTED
    assert L.vq_gemv(d, FAKE + 2, 1, 1, FAKE, None) == VQ_ERR_ALIGN
    assert L.vq_gemv(d, FAKE, 0, 1, FAKE + 4, None) == VQ_ERR_ALIGN


def test_gemm_argument_checks(L):
    d = ctypes.byref(fake_desc())
    assert L.vq_gemm(d, None, 4, FAKE, None, 0, None) == VQ_ERR_NULL
    assert L.vq_gemm(d, FAKE, 4, None, None, 0, None) == VQ_ERR_NULL
    assert L.vq_gemm(d, FAKE, 0, FAKE, None, 0, None) == VQ_ERR_SHAPE
    assert L.vq_gemm(d, FAKE, 1 << 30, FAKE, None, 0, None) == VQ_ERR_SHAPE
    assert L.vq_gemm(d, FAKE + 2, 4, FAKE, None, 0, None) == VQ_ERR_ALIGN
    assert L.vq_gemm(d, FAKE, 4, FAKE, None, 64, None) == VQ_ERR_NULL      # bytes without a buffer
    assert L.vq_gemm(d, FAKE, 4, FAKE, FAKE + 8, 64, None) == VQ_ERR_ALIGN


@pytest.mark.parametrize("n,k,bits,stages,m", [(64, 64, 12, 1, 4), (4096, 4096, 12, 2, 2048), (14336, 4096, 12, 2, 2048),
                                               (4096, 4096, 12, 2, 1), (28672, 8192, 16, 1, 64), (256, 512, 8, 1, 40)])
def test_gemm_workspace_contract(L, n, k, bits, stages, m):
    """vq_gemm takes any workspace of at least vq_gemm_workspace_size bytes
    and returns VQ_ERR_WORKSPACE, before any HIP call, for one byte less."""
    d = ctypes.byref(fake_desc(n=n, k=k, bits=bits, stages=stages, bs=128))
    need = L.vq_gemm_workspace_size(d, m)
    assert need % 256 == 0
    if need:
        assert L.vq_gemm(d, FAKE, m, FAKE, FAKE, need - 1, None) == VQ_ERR_WORKSPACE
        assert L.vq_gemm(d, FAKE, m, FAKE, None, 0, None) == VQ_ERR_WORKSPACE


def test_gemm_noalloc_checks(L):
    """The no-allocation entry point validates like vq_gemm and refuses,
    before any HIP call, a call that needs more than its static scratch."""
    d = ctypes.byref(fake_desc(n=4096, k=4096, bits=12, stages=2, bs=128))
    assert L.vq_gemm_noalloc(d, None, 2048, FAKE, None) == VQ_ERR_NULL
    assert L.vq_gemm_noalloc(d, FAKE, 0, FAKE, None) == VQ_ERR_SHAPE
    assert L.vq_gemm_noalloc(d, FAKE + 2, 2048, FAKE, None) == VQ_ERR_ALIGN
    limit = 33 << 20
    m_big = 8192  # 8192 tokens x 4096 columns of fp16 x: 64 MiB of scratch
    assert L.vq_gemm_workspace_size(d, m_big) > limit
    assert L.vq_gemm_noalloc(d, FAKE, m_big, FAKE, None) == VQ_ERR_WORKSPACE
    assert L.vq_gemm_workspace_size(d, 4096) <= limit
    bad = fake_desc()
    bad.n_out = 0
    assert L.vq_gemm_noalloc(ctypes.byref(bad), FAKE, 64, FAKE, None) == VQ_ERR_SHAPE


def test_header_states_noalloc_limit():
    m = re.search(r"#define VQ_GEMM_NOALLOC_SCRATCH \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == 33 << 20


def test_gemm_workspace_size_invalid(L):
    assert L.vq_gemm_workspace_size(None, 16) == 0
    d = fake_desc()
    assert L.vq_gemm_workspace_size(ctypes.byref(d), 0) == 0
    d.n_out = 0
    assert L.vq_gemm_workspace_size(ctypes.byref(d), 16) == 0


def test_gemv_rht_argument_checks(L):
    """The fused input transform: argument errors, and VQ_ERR_UNSUPPORTED
    (nothing launched) for weights the 16-bit decode kernel does not take."""
    d16 = ctypes.byref(fake_desc(n=64, k=4096, bits=16, bs=128))
    assert L.vq_gemv_rht(d16, None, 1, 1, FAKE, 64, FAKE, None) == VQ_ERR_NULL
    assert L.vq_gemv_rht(d16, FAKE, 1, 1, None, 64, FAKE, None) == VQ_ERR_NULL
    assert L.vq_gemv_rht(d16, FAKE, 1, 1, FAKE, 64, None, None) == VQ_ERR_NULL
    assert L.vq_gemv_rht(d16, FAKE, 7, 1, FAKE, 64, FAKE, None) == VQ_ERR_DTYPE
    assert L.vq_gemv_rht(d16, FAKE, 1, 0, FAKE, 64, FAKE, None) == VQ_ERR_UNSUPPORTED
    assert L.vq_gemv_rht(d16, FAKE, 1, 17, FAKE, 64, FAKE, None) == VQ_ERR_UNSUPPORTED
    for mb in (0, 48, 32768):
        assert L.vq_gemv_rht(d16, FAKE, 1, 1, FAKE, mb, FAKE, None) == VQ_ERR_SHAPE
    assert L.vq_gemv_rht(d16, FAKE, 1, 1, FAKE + 4, 64, FAKE, None) == VQ_ERR_ALIGN
    assert L.vq_gemv_rht(d16, FAKE + 2, 1, 1, FAKE, 64, FAKE, None) == VQ_ERR_ALIGN
    for desc in (fake_desc(n=64, k=4096, bits=12, bs=128),            # 12-bit indices
                 fake_desc(n=64, k=4000, bits=16, bs=32),             # K % 2048
                 fake_desc(n=64, k=34816, bits=16, bs=128),           # K past 32768
                 fake_desc(n=64, k=28672, stages=2, bits=16, bs=128),  # 16 + 16 past 26624
                 fake_desc(n=64, k=4096, bits=16, bs=96),             # scale block not dividing 2048
                 fake_desc(n=64, k=4096, stages=3, bits=16, bs=128)):  # three stages
        assert L.vq_gemv_rht(ctypes.byref(desc), FAKE, 1, 1, FAKE, 64, FAKE, None) == VQ_ERR_UNSUPPORTED
    sp = fake_desc(n=64, k=4096, bits=16, bs=128)  # a sparse correction: not taken either
    sp.sp_nnz = 5
    sp.sp_rowptr, sp.sp_col, sp.sp_val = FAKE, FAKE, FAKE
    assert L.vq_validate(ctypes.byref(sp)) == 0
    assert L.vq_gemv_rht(ctypes.byref(sp), FAKE, 1, 1, FAKE, 64, FAKE, None) == VQ_ERR_UNSUPPORTED


def test_unpack_argument_checks(L):
    d = ctypes.byref(fake_desc())
    assert L.vq_unpack_dequant(d, None, None, None) == VQ_ERR_NULL
    assert L.vq_unpack_dequant(d, FAKE + 2, None, None) == VQ_ERR_ALIGN
    assert L.vq_unpack_dequant(d, None, FAKE + 8, None) == VQ_ERR_ALIGN


def test_rht_argument_checks(L):
    assert L.rht_apply(None, 0, 1, 64, FAKE, 64, FAKE, None) == VQ_ERR_NULL
    assert L.rht_apply(FAKE, 0, 1, 64, None, 64, FAKE, None) == VQ_ERR_NULL
    assert L.rht_apply(FAKE, 0, 1, 64, FAKE, 64, None, None) == VQ_ERR_NULL
    assert L.rht_apply(FAKE, 5, 1, 64, FAKE, 64, FAKE, None) == VQ_ERR_DTYPE
    assert L.rht_apply(FAKE, 0, 0, 64, FAKE, 64, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply(FAKE, 0, 1, 0, FAKE, 64, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply(FAKE, 0, 1, 64, FAKE, 48, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply(FAKE, 0, 1, 64, FAKE, 32768, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply(FAKE, 0, 1, 64, FAKE, 0, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply(FAKE + 4, 0, 1, 64, FAKE, 64, FAKE, None) == VQ_ERR_ALIGN


def _lens(*v):
    arr = (ctypes.c_int32 * len(v))(*v)
    return ctypes.cast(arr, ctypes.c_void_p), arr


def test_rht_shards_argument_checks(L):
    """Shard lists are checked on the host: positive lengths that sum to n,
    1..16 shards, a known direction; nothing is launched on an error."""
    ok, _k1 = _lens(48, 16)
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 2, None, FAKE, 64, 0, FAKE, None) == VQ_ERR_NULL
    assert L.rht_apply_shards(None, 0, 1, 64, 2, ok, FAKE, 64, 0, FAKE, None) == VQ_ERR_NULL
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 2, ok, None, 64, 0, FAKE, None) == VQ_ERR_NULL
    assert L.rht_apply_shards(FAKE, 3, 1, 64, 2, ok, FAKE, 64, 0, FAKE, None) == VQ_ERR_DTYPE
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 2, ok, FAKE, 64, 2, FAKE, None) == VQ_ERR_VALUE
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 0, ok, FAKE, 64, 0, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 17, ok, FAKE, 64, 0, FAKE, None) == VQ_ERR_SHAPE
    short, _k2 = _lens(48, 8)
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 2, short, FAKE, 64, 1, FAKE, None) == VQ_ERR_SHAPE
    neg, _k3 = _lens(80, -16)
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 2, neg, FAKE, 64, 1, FAKE, None) == VQ_ERR_SHAPE
    zero, _k4 = _lens(64, 0)
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 2, zero, FAKE, 64, 1, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply_shards(FAKE, 0, 1, 64, 2, ok, FAKE, 96, 1, FAKE, None) == VQ_ERR_SHAPE
    assert L.rht_apply_shards(FAKE + 4, 0, 1, 64, 2, ok, FAKE, 64, 1, FAKE, None) == VQ_ERR_ALIGN


def test_header_rht_constants():
    src = open(HEADER).read()
    import compressed_index_matmul_amd as vq
    assert re.search(r"#define VQ_RHT_FORWARD 0\b", src) and re.search(r"#define VQ_RHT_INVERSE 1\b", src)
    assert int(re.search(r"#define VQ_RHT_MAX_SHARDS (\d+)", src).group(1)) == vq.VQ_RHT_MAX_SHARDS


@pytest.mark.parametrize("wl", [w for w in vqsynth.WORKLOADS if isinstance(vqsynth.WORKLOADS[w]["bits"], int)])
def test_compressed_bytes_match_oracle(L, wl):
    """The library's byte count equals the oracle's closed form for every
    workload shape (two independent implementations of the same arithmetic)."""
    cfg = vqsynth.WORKLOADS[wl]
    for _, n, k in cfg["shapes"]:
        bs = k if cfg["scale_block"] is None else cfg["scale_block"]
        d = fake_desc(n, k, cfg["stages"], cfg["bits"], bs)
        assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(n, k, cfg["stages"], cfg["bits"], bs)


@pytest.mark.parametrize("n,k,st,bits,bs", [(3, 24, 1, 12, 24), (5, 72, 2, 12, 16), (1, 8, 4, 8, 8), (7, 40, 3, 16, 4096)])
def test_compressed_bytes_ragged(L, n, k, st, bits, bs):
    d = fake_desc(n, k, st, bits, bs)
    assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(n, k, st, bits, min(bs, k) if bs > k else bs)


@pytest.mark.parametrize("widths", [[12, 4], [8, 4], [16, 8], [16, 16, 8], [16, 16, 16, 8], [4], [4, 4, 4, 4],
                                    [12, 12, 4], [16, 12, 8, 4]])
def test_valid_ladders(L, widths):
    d = fake_desc(stages=len(widths), widths=widths)
    assert L.vq_validate(ctypes.byref(d)) == VQ_OK
    d = fake_desc(stages=len(widths), widths=widths, stage_scales=[1.0, 0.25, -3.0, 1e-30][:len(widths)])
    assert L.vq_validate(ctypes.byref(d)) == VQ_OK


def test_stage_bits_zero_means_idx_bits(L):
    d = fake_desc(stages=2, bits=16)          # stage_bits all 0 -> 16, 16
    assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(64, 64, 2, 16, 32)
    d.stage_bits[1] = 8                        # 16 + 8 now needs idx_lo[1]
    assert L.vq_validate(ctypes.byref(d)) == VQ_ERR_NULL
    d.idx_lo[1] = FAKE
    assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(64, 64, 2, [16, 8], 32)


@pytest.mark.parametrize("mutate,code", [
    (lambda d: d.stage_bits.__setitem__(1, 6), VQ_ERR_UNSUPPORTED),
    (lambda d: d.stage_bits.__setitem__(0, 32), VQ_ERR_UNSUPPORTED),
    (lambda d: d.idx_hi.__setitem__(1, None), VQ_ERR_NULL),          # 4-bit stage without its nibble plane
    (lambda d: d.idx_hi.__setitem__(1, FAKE + 1), VQ_ERR_ALIGN),
    (lambda d: d.idx_lo.__setitem__(0, None), VQ_ERR_NULL),
    (lambda d: setattr(d, "flags", 2), VQ_ERR_UNSUPPORTED),
    (lambda d: (setattr(d, "flags", 1), d.stage_scale.__setitem__(1, float("inf"))), VQ_ERR_VALUE),
    (lambda d: (setattr(d, "flags", 1), d.stage_scale.__setitem__(0, float("nan"))), VQ_ERR_VALUE),
])
def test_invalid_ladder(L, mutate, code):
    d = fake_desc(stages=2, widths=[12, 4])
    mutate(d)
    assert L.vq_validate(ctypes.byref(d)) == code
    assert L.vq_gemv(ctypes.byref(d), FAKE, 1, 1, FAKE, None) == code
    assert L.vq_gemm(ctypes.byref(d), FAKE, 64, FAKE, None, 0, None) == code
    assert L.vq_unpack_dequant(ctypes.byref(d), FAKE, FAKE, None) == code


def test_unused_stage_fields_ignored(L):
    d = fake_desc(stages=2, widths=[12, 4])
    d.stage_bits[3] = 7                        # beyond n_stages
    d.stage_scale[1] = float("inf")            # no VQ_STAGE_SCALES flag
    assert L.vq_validate(ctypes.byref(d)) == VQ_OK
    d.flags = 1
    d.stage_scale[1] = 0.5
    d.stage_scale[2] = float("nan")            # beyond n_stages
    assert L.vq_validate(ctypes.byref(d)) == VQ_OK


@pytest.mark.parametrize("n,k,widths,bs", [(576, 576, [12, 4], 128), (3, 24, [12, 4], 24), (5, 40, [4], 8),
                                           (7, 72, [16, 8], 72), (1, 8, [16, 16, 16, 8], 8), (9, 88, [8, 4, 12], 16)])
def test_compressed_bytes_ladders(L, n, k, widths, bs):
    d = fake_desc(n, k, len(widths), widths[0], bs, widths=widths)
    assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(n, k, len(widths), widths, bs)


@pytest.mark.parametrize("wl", ["smollm_rvq124", "llama8b_rvq124", "mlp70b_e8p3"])
def test_ladder_workload_bytes(L, wl):
    cfg = vqsynth.WORKLOADS[wl]
    for _, n, k in cfg["shapes"]:
        bs = k if cfg["scale_block"] is None else cfg["scale_block"]
        d = fake_desc(n, k, cfg["stages"], cfg["bits"][0], bs, widths=list(cfg["bits"]))
        assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(n, k, cfg["stages"], list(cfg["bits"]), bs)


def sparse_desc(nnz=5, **kw):
    d = fake_desc(**kw)
    d.sp_nnz = nnz
    d.sp_rowptr, d.sp_col, d.sp_val = FAKE, FAKE, FAKE
    return d


def test_sparse_correction_fields(L):
    d = sparse_desc()
    assert L.vq_validate(ctypes.byref(d)) == VQ_OK
    n, k = d.n_out, d.k_in
    assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(n, k, 1, 12, 32, sparse_nnz=5)
    # nnz == 0: the pointers are ignored
    d = fake_desc()
    d.sp_rowptr = FAKE + 3
    assert L.vq_validate(ctypes.byref(d)) == VQ_OK


@pytest.mark.parametrize("mutate,code", [
    (lambda d: setattr(d, "sp_nnz", -1), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "sp_reserved", 1), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "sp_rowptr", None), VQ_ERR_NULL),
    (lambda d: setattr(d, "sp_col", None), VQ_ERR_NULL),
    (lambda d: setattr(d, "sp_val", None), VQ_ERR_NULL),
    (lambda d: setattr(d, "sp_col", FAKE + 4), VQ_ERR_ALIGN),
    (lambda d: setattr(d, "sp_val", FAKE + 2), VQ_ERR_ALIGN),
])
def test_invalid_sparse(L, mutate, code):
    d = sparse_desc()
    mutate(d)
    assert L.vq_validate(ctypes.byref(d)) == code
    assert L.vq_gemv(ctypes.byref(d), FAKE, 1, 1, FAKE, None) == code
    assert L.vq_gemm(ctypes.byref(d), FAKE, 64, FAKE, None, 0, None) == code
    assert L.vq_unpack_dequant(ctypes.byref(d), FAKE, FAKE, None) == code


def test_sparse_bytes_by_hand():
    # 3 rows, 2 entries: 4 int32 row pointers + 2 int32 columns + 2 fp16 values
    base = oracle.compressed_bytes(3, 16, 1, 8, 16)
    assert oracle.compressed_bytes(3, 16, 1, 8, 16, sparse_nnz=2) == base + 16 + 8 + 4


def lowrank_desc(rank=16, n=64, k=64):
    d = fake_desc(n=n, k=k)
    d.lr_rank, d.lr_u, d.lr_v = rank, FAKE, FAKE
    return d


def test_valid_lowrank(L):
    for rank in (1, 7, 256):
        assert L.vq_validate(ctypes.byref(lowrank_desc(rank))) == VQ_OK
    d = fake_desc()
    d.lr_u = FAKE + 3  # rank 0: the pointers are ignored
    assert L.vq_validate(ctypes.byref(d)) == VQ_OK


@pytest.mark.parametrize("mutate,code", [
    (lambda d: setattr(d, "lr_rank", -1), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "lr_rank", 257), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "lr_reserved", 1), VQ_ERR_SHAPE),
    (lambda d: setattr(d, "lr_u", None), VQ_ERR_NULL),
    (lambda d: setattr(d, "lr_v", None), VQ_ERR_NULL),
    (lambda d: setattr(d, "lr_u", FAKE + 2), VQ_ERR_ALIGN),
    (lambda d: setattr(d, "lr_v", FAKE + 8), VQ_ERR_ALIGN),
])
def test_invalid_lowrank(L, mutate, code):
    d = lowrank_desc()
    mutate(d)
    assert L.vq_validate(ctypes.byref(d)) == code
    assert L.vq_gemv(ctypes.byref(d), FAKE, 1, 1, FAKE, None) == code
    assert L.vq_gemm(ctypes.byref(d), FAKE, 64, FAKE, None, 0, None) == code
    assert L.vq_gemm_noalloc(ctypes.byref(d), FAKE, 64, FAKE, None) == code
    assert L.vq_unpack_dequant(ctypes.byref(d), FAKE, FAKE, None) == code


@pytest.mark.parametrize("rank", [1, 32, 256])
def test_lowrank_bytes_match_oracle(L, rank):
    d = lowrank_desc(rank, n=4096, k=14336)
    d.scale_block = 128
    assert L.vq_compressed_bytes(ctypes.byref(d)) == oracle.compressed_bytes(4096, 14336, 1, 12, 128,
                                                                             lowrank_rank=rank)


def test_lowrank_workspace(L):
    """The many-token product keeps t = x V^T (m x rank floats) in the
    workspace after the main product's part, so even the bf16 path (64
    tokens or fewer) needs one; too little is refused before any HIP call."""
    d = lowrank_desc(32, n=4096, k=4096)
    d.n_stages, d.scale_block = 2, 128
    for t in range(2):
        d.codebook[t], d.idx_lo[t], d.idx_hi[t] = FAKE, FAKE, FAKE
    plain = fake_desc(n=4096, k=4096, stages=2, bits=12, bs=128)
    for m in (1, 40, 300, 2048):
        extra = (m * 32 * 4 + 255) // 256 * 256
        assert L.vq_gemm_workspace_size(ctypes.byref(d), m) == L.vq_gemm_workspace_size(ctypes.byref(plain), m) + extra
        need = L.vq_gemm_workspace_size(ctypes.byref(d), m)
        assert L.vq_gemm(ctypes.byref(d), FAKE, m, FAKE, FAKE, need - 256, None) == VQ_ERR_WORKSPACE


def test_gemv_rht_refuses_lowrank(L):
    d = fake_desc(n=8192, k=4096, bits=16, bs=4096)
    d.lr_rank, d.lr_u, d.lr_v = 8, FAKE, FAKE
    assert L.vq_gemv_rht(ctypes.byref(d), FAKE, 1, 1, FAKE, 4096, FAKE, None) == VQ_ERR_UNSUPPORTED
