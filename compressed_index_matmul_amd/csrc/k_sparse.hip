// Sparse correction of the products: y[b][r] += sum_j val_j x[b][col_j] over
// the correction's row r (orka README, "How it works": the decoded weight
// plus a sparse correction), launched after the main product on the same
// stream.  CSR over output rows; fp16 values, fp32 products and sums in a
// fixed order (no atomics).
//
// Up to 8 tokens: one wave per row, lanes split the row's entries, one wave
// sum per token.
// 9 to 64 tokens: a wave takes a row and a block of 16 tokens, lane =
// (entry slot e = lane / 16, token lane % 16); slot e takes the row's
// entries e, e + 4, ... in storage order, and the four slots are added
// across lanes in a fixed order.  Where a token block's x fits in 8 KiB per
// token (bf16 K <= 4096, fp32 K <= 2048), a workgroup of rows first copies
// it into LDS (rows padded by 16 bytes, so the 16 tokens of one column fall
// in distinct banks) and reads x there (k_sparse_lds); otherwise each lane
// gathers its x value from global memory (k_sparse_mid).
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

constexpr int kSpRowBytes = 8192;            // x bytes per token row that k_sparse_lds takes
constexpr int kSpPitch = kSpRowBytes + 16;   // LDS bytes per token row
constexpr int kSpWaves = 16;

// A row's entries base .. base + 63 (those below hi), one per lane: the
// column (-1: none) and the fp16 value bits.
struct SpEnt {
  int c;
  uint32_t v;
};

// tokens 16 blockIdx.y .. + 15 (those below m), K * sizeof(x) <= kSpRowBytes;
// a workgroup takes rows_per_wg rows
__global__ __launch_bounds__(kSpWaves * 64) void k_sparse_lds(SparseArgs a, int rows_per_wg) {
  __shared__ __attribute__((aligned(16))) uint8_t s_x[16 * kSpPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r_lo = blockIdx.x * rows_per_wg;
  const int r_hi = min(a.n, r_lo + rows_per_wg);
  if (r_lo >= r_hi) return;  // whole workgroup, before any barrier
  const int xb = a.xt == VQ_F32 ? 4 : 2;
  const int e = lane >> 4;
  const int b = 16 * blockIdx.y + (lane & 15);
  const uint8_t *xrow = s_x + (lane & 15) * kSpPitch;
  auto load_ent = [&](int base, int hi) {
    SpEnt t{-1, 0u};
    const int j = base + lane;
    if (j < hi) {
      t.c = a.col[j];
      t.v = a.val[j];
    }
    return t;
  };
  // the wave's first row's first 64 entries load while x is staged
  int r = r_lo + wave;
  int lo = 0, hi = 0;
  SpEnt cur{-1, 0u};
  if (r < r_hi) {
    sp_range(a, r, lo, hi);
    cur = load_ent(lo, hi);
  }
  // x[16 block tokens][0, K) into LDS (tokens past m: the last one)
  const int pieces = a.k * xb / 16;  // 16-byte pieces per token row (K % 8 == 0)
  if (pieces % 64 == 0) {
    // LDS-direct loads: a wave moves 1 KiB pieces of one token row
    for (int q = wave; q < 16 * pieces / 64; q += kSpWaves) {
      const int t = 64 * q / pieces, pc0 = 64 * q - t * pieces;
      const int tok = min(16 * (int)blockIdx.y + t, a.m - 1);
      lds_direct_16(reinterpret_cast<const uint8_t *>(a.x) + (size_t)tok * a.k * xb + 16 * (pc0 + lane),
                    s_x + t * kSpPitch + 16 * pc0);
    }
  } else {
    for (int i = tid; i < 16 * pieces; i += kSpWaves * 64) {
      const int t = i / pieces, pc = i - t * pieces;
      const int tok = min(16 * (int)blockIdx.y + t, a.m - 1);
      *reinterpret_cast<uint4 *>(s_x + t * kSpPitch + 16 * pc) =
          reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(a.x) + (size_t)tok * a.k * xb)[pc];
    }
  }
  wait_all_memory();  // the LDS-direct loads have landed
  __syncthreads();
  for (; r < r_hi; r += kSpWaves) {
    float acc = 0.f;
    int base = lo;
    for (;;) {  // 64 entries of row r at a time (wave-uniform control)
      // prefetch the row's next 64 entries, else the wave's next row's first
      const bool more = base + 64 < hi;
      int nlo = 0, nhi = 0;
      if (!more && r + kSpWaves < r_hi) sp_range(a, r + kSpWaves, nlo, nhi);
      const SpEnt nxt = more ? load_ent(base + 64, hi) : load_ent(nlo, nhi);
      const int cnt = min(64, hi - base);  // <= 0 for a row without entries
      for (int it = 0; it < cnt; it += 4) {  // slot e: entry it + e, storage order
        const int src = it + e;
        const int c = __shfl(cur.c, src);
        const uint32_t v = (uint32_t)__shfl((int)cur.v, src);
        if (src < cnt && c >= 0 && c < a.k) {
          const float xv = xb == 4 ? *reinterpret_cast<const float *>(xrow + 4 * c)
                                   : bf2f(*reinterpret_cast<const uint16_t *>(xrow + 2 * c));
          acc = fmaf(h2f(v), xv, acc);
        }
      }
      cur = nxt;
      if (more) {
        base += 64;
        continue;
      }
      lo = nlo;  // the range of row r + kSpWaves
      hi = nhi;
      break;
    }
    acc += __shfl_xor(acc, 16);  // slots (0 + 1), (2 + 3)
    acc += __shfl_xor(acc, 32);  // then their sum
    if (e == 0 && b < a.m) a.y[(size_t)b * a.n + r] += acc;
  }
}

hipError_t launch_sparse_add(const WView &w, const void *x, int xt, int m, float *y, hipStream_t s) {
  if (w.sp_nnz <= 0) return hipSuccess;
  SparseArgs a{w.sp_rowptr, w.sp_col, w.sp_val, x, y, w.sp_nnz, w.n, w.k, m, xt};
  if (m <= 64) {
    const unsigned blocks = (unsigned)((w.n + 3) / 4);
    if (m <= 1) hipLaunchKernelGGL(k_sparse_few<1>, dim3(blocks), dim3(256), 0, s, a);
    else if (m <= 4) hipLaunchKernelGGL(k_sparse_few<4>, dim3(blocks), dim3(256), 0, s, a);
    else if (m <= 8) hipLaunchKernelGGL(k_sparse_few<8>, dim3(blocks), dim3(256), 0, s, a);
    else if ((int64_t)w.k * (xt == VQ_F32 ? 4 : 2) <= kSpRowBytes) {  // a token block's x fits LDS
      const int cus = device_cu_count();
      const int grid = min((w.n + kSpWaves - 1) / kSpWaves, cus);
      const int rows = (w.n + grid - 1) / grid;
      hipLaunchKernelGGL(k_sparse_lds, dim3((unsigned)grid, (unsigned)((m + 15) / 16)), dim3(kSpWaves * 64), 0, s, a,
                         rows);
    } else {
      hipLaunchKernelGGL(k_sparse_mid, dim3(blocks, (unsigned)((m + 15) / 16)), dim3(256), 0, s, a);
    }
  } else {
    const int64_t items = (int64_t)w.n * ((m + 63) / 64);
    hipLaunchKernelGGL(k_sparse_many, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace vqmm
