// Standalone bit-plane unpack + exact dequant to fp16 (orka README, "How it
// works": indices stored as a low-byte plane plus packed high nibbles; a
// group decodes to scale x sum of its stages' codebook entries).
//
// One thread per group.  The stage sum and the product with the scale are
// formed in float64, where they are exact (at most four fp16 terms and an
// fp16 factor need < 53 significant bits), and rounded once to fp16 with
// integer arithmetic on the bit pattern, so the result is the correctly
// rounded value whatever the summation order.  Write-bandwidth bound.  A
// sparse correction (orka README, "How it works": the decode plus a sparse
// correction) is added to the float64 value entry by entry, in storage
// order, before the one rounding.
//
// Residual ladders (per-stage widths) and stage scales (GLQ page, "Inference
// kernels": the inverse residual scale of the two-stage call) take the
// BITS = 0 instantiation: each stage's width is read at run time, each
// entry is multiplied by its stage scale in float64 (exact: 24 + 11
// significant bits), the products are added from stage 0 up with float64
// rounding and the sum is multiplied by the block scale in float64 -- a
// fixed order, so the fp16 result is reproducible bit for bit.
#include "vqmm_device.h"
#include "vqmm_internal.h"

namespace vqmm {

struct DequantArgs {
  const uint8_t *lo[VQ_MAX_STAGES];
  const uint8_t *hi[VQ_MAX_STAGES];
  const uint16_t *i16[VQ_MAX_STAGES];
  const uint16_t *cb[VQ_MAX_STAGES];
  const uint16_t *sc;
  uint16_t *idx_out;  // [S][N*G] or null
  uint16_t *w_out;    // [N][K] or null
  int64_t total;      // N * G
  int G, S, bits, bs, nblk, k;
  int sb[VQ_MAX_STAGES];    // index width of each stage
  float rs[VQ_MAX_STAGES];  // stage scales
  int sp_nnz;               // sparse correction (CSR over rows), 0 = none
  const int32_t *sp_rowptr;
  const int32_t *sp_col;
  const uint16_t *sp_val;
};

// BITS: the width of every stage, or 0 for per-stage widths and scales.
template <int BITS>
__global__ __launch_bounds__(256) void k_unpack_dequant(DequantArgs a) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= a.total) return;
  const int64_t r = f / a.G;
  const int g = (int)(f - r * a.G);
  double acc[8];
  for (int t = 0; t < a.S; ++t) {
    uint32_t idx = load_index(BITS ? BITS : a.sb[t], a.lo[t], a.hi[t], a.i16[t], (size_t)f);
    if (a.idx_out) a.idx_out[(int64_t)t * a.total + f] = (uint16_t)idx;
    if (a.w_out) {
      const uint4 v = reinterpret_cast<const uint4 *>(a.cb[t])[idx];
      const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double c = (double)h2f((h[j >> 1] >> ((j & 1) * 16)) & 0xffffu);
        if (BITS == 0) c *= (double)a.rs[t];  // exact product
        acc[j] = (t == 0) ? c : acc[j] + c;  // sum starts at stage 0
      }
    }
  }
  if (!a.w_out) return;
  const double s = (double)h2f(a.sc[r * a.nblk + (8 * g) / a.bs]);
  double wv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wv[j] = s * acc[j];
  if (a.sp_nnz > 0) {
    // entries of row r in this group's columns: lower bound of column 8g in
    // the row's ascending columns, then forward in storage order (each
    // addition rounded to float64); the row range is clamped to the arrays
    const int lo = min(max(a.sp_rowptr[r], 0), a.sp_nnz);
    const int hi = min(max(a.sp_rowptr[r + 1], lo), a.sp_nnz);
    int b0 = lo, b1 = hi;
    while (b0 < b1) {
      const int mid = (b0 + b1) >> 1;
      if (a.sp_col[mid] < 8 * g) b0 = mid + 1;
      else b1 = mid;
    }
    for (int j = b0; j < hi; ++j) {
      const int c = a.sp_col[j] - 8 * g;
      if (c >= 8) break;
      if (c < 0) continue;
      const double v = (double)h2f(a.sp_val[j]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q == c) wv[q] = wv[q] + v;
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f64_to_f16_rne(wv[2 * j]) | (f64_to_f16_rne(wv[2 * j + 1]) << 16);
  reinterpret_cast<uint4 *>(a.w_out + r * (int64_t)a.k)[g] = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_unpack_dequant(const WView &w, uint16_t *idx_out, uint16_t *w_out, hipStream_t s) {
  DequantArgs a{};
  for (int t = 0; t < VQ_MAX_STAGES; ++t) {
    a.lo[t] = w.lo[t];
    a.hi[t] = w.hi[t];
    a.i16[t] = w.i16[t];
    a.cb[t] = w.cb[t];
  }
  a.sc = w.sc;
  a.idx_out = idx_out;
  a.w_out = w_out;
  a.total = (int64_t)w.n * w.G;
  a.G = w.G;
  a.S = w.S;
  a.bits = w.bits;
  a.bs = w.bs;
  a.nblk = w.nblk;
  a.k = w.k;
  for (int t = 0; t < VQ_MAX_STAGES; ++t) {
    a.sb[t] = t < w.S ? w.sb[t] : 0;
    a.rs[t] = w.rs[t];
  }
  a.sp_nnz = w.sp_nnz;
  a.sp_rowptr = w.sp_rowptr;
  a.sp_col = w.sp_col;
  a.sp_val = w.sp_val;
  const unsigned blocks = (unsigned)((a.total + 255) / 256);
  if (!plain_format(w))
    hipLaunchKernelGGL(k_unpack_dequant<0>, dim3(blocks), dim3(256), 0, s, a);
  else if (w.bits == 8)
    hipLaunchKernelGGL(k_unpack_dequant<8>, dim3(blocks), dim3(256), 0, s, a);
  else if (w.bits == 12)
    hipLaunchKernelGGL(k_unpack_dequant<12>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_unpack_dequant<16>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace vqmm
