// Sparse correction of the products: y[b][r] += sum_j val_j x[b][col_j] over
// the correction's row r (orka README, "How it works": the decoded weight
// plus a sparse correction), launched after the main product on the same
// stream.  CSR over output rows; fp16 values, fp32 products and sums in a
// fixed order (no atomics).
//
// Up to 8 tokens: one wave per row, lanes split the row's entries, one wave
// sum per token.
// 9 to 64 tokens: one wave per (row, block of 16 tokens); lane = (entry
// slot e = lane / 16, token lane % 16), slot e takes entries e, e + 4, ...
// of the row in storage order, and the four slots are added in a fixed
// order across lanes.
// More tokens: one wave per (row, 64 tokens), lane = token, the row's
// entries in storage order (value and column are wave-uniform loads).  The
// decode kernel fuses the correction itself where it runs; this launch
// serves the other paths.  Row ranges are clamped to [0, nnz] and columns past
// the row are skipped, so inconsistent CSR data stays inside its arrays.
#include "vqmm_device.h"
#include "vqmm_internal.h"

namespace vqmm {

struct SparseArgs {
  const int32_t *rowptr;
  const int32_t *col;
  const uint16_t *val;
  const void *x;  // [m][k], fp32 or bf16
  float *y;       // [m][n]
  int nnz, n, k, m, xt;
};

__device__ __forceinline__ float sp_x(const SparseArgs &a, int b, int c) {
  const size_t i = (size_t)b * a.k + c;
  return a.xt == VQ_F32 ? reinterpret_cast<const float *>(a.x)[i] : bf2f(reinterpret_cast<const uint16_t *>(a.x)[i]);
}

__device__ __forceinline__ void sp_range(const SparseArgs &a, int r, int &lo, int &hi) {
  lo = min(max(a.rowptr[r], 0), a.nnz);
  hi = min(max(a.rowptr[r + 1], lo), a.nnz);
}

template <int MT>
__global__ __launch_bounds__(256) void k_sparse_few(SparseArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= a.n) return;
  int lo, hi;
  sp_range(a, r, lo, hi);
  float acc[MT];
#pragma unroll
  for (int b = 0; b < MT; ++b) acc[b] = 0.f;
  for (int j = lo + lane; j < hi; j += 64) {
    const int c = a.col[j];
    if (c < 0 || c >= a.k) continue;
    const float v = h2f(a.val[j]);
#pragma unroll
    for (int b = 0; b < MT; ++b)
      if (b < a.m) acc[b] = fmaf(v, sp_x(a, b, c), acc[b]);
  }
#pragma unroll
  for (int b = 0; b < MT; ++b) {
    if (b < a.m) {
      const float t = wave_sum(acc[b]);
      if (lane == 0) a.y[(size_t)b * a.n + r] += t;
    }
  }
}

// tokens 16 blockIdx.y .. + 15 (those below m)
__global__ __launch_bounds__(256) void k_sparse_mid(SparseArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= a.n) return;
  const int e = lane >> 4;
  const int b = 16 * blockIdx.y + (lane & 15);
  const int bc = min(b, a.m - 1);  // tokens past m load a valid row, never stored
  int lo, hi;
  sp_range(a, r, lo, hi);
  float acc = 0.f;
  for (int j = lo + e; j < hi; j += 4) {
    const int c = a.col[j];
    if (c >= 0 && c < a.k) acc = fmaf(h2f(a.val[j]), sp_x(a, bc, c), acc);
  }
  acc += __shfl_xor(acc, 16);  // slots (0 + 1), (2 + 3)
  acc += __shfl_xor(acc, 32);  // then their sum
  if (e == 0 && b < a.m) a.y[(size_t)b * a.n + r] += acc;
}

__global__ __launch_bounds__(256) void k_sparse_many(SparseArgs a) {
  const int lane = threadIdx.x & 63;
  const int tb = (a.m + 63) / 64;
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= a.n * tb) return;
  const int r = item / tb;
  const int b = (item - r * tb) * 64 + lane;
  int lo, hi;
  sp_range(a, r, lo, hi);
  float acc = 0.f;
  for (int j = lo; j < hi; ++j) {
    const int c = a.col[j];
    if (c < 0 || c >= a.k) continue;
    if (b < a.m) acc = fmaf(h2f(a.val[j]), sp_x(a, b, c), acc);
  }
  if (b < a.m) a.y[(size_t)b * a.n + r] += acc;
}

hipError_t launch_sparse_add(const WView &w, const void *x, int xt, int m, float *y, hipStream_t s) {
  if (w.sp_nnz <= 0) return hipSuccess;
  SparseArgs a{w.sp_rowptr, w.sp_col, w.sp_val, x, y, w.sp_nnz, w.n, w.k, m, xt};
  if (m <= 64) {
    const unsigned blocks = (unsigned)((w.n + 3) / 4);
    if (m <= 1) hipLaunchKernelGGL(k_sparse_few<1>, dim3(blocks), dim3(256), 0, s, a);
    else if (m <= 4) hipLaunchKernelGGL(k_sparse_few<4>, dim3(blocks), dim3(256), 0, s, a);
    else if (m <= 8) hipLaunchKernelGGL(k_sparse_few<8>, dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_sparse_mid, dim3(blocks, (unsigned)((m + 15) / 16)), dim3(256), 0, s, a);
  } else {
    const int64_t items = (int64_t)w.n * ((m + 63) / 64);
    hipLaunchKernelGGL(k_sparse_many, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace vqmm
