// Standalone bit-plane unpack + exact dequant to fp16 (orka README, "How it
// works": indices stored as a low-byte plane plus packed high nibbles; a
// group decodes to scale x sum of its stages' codebook entries).
//
// One thread per group.  The stage sum and the product with the scale are
// formed in float64, where they are exact (at most four fp16 terms and an
// fp16 factor need < 53 significant bits), and rounded once to fp16 (round
// to odd into float, then the hardware conversion; see round_group_f16),
// so the result is the correctly rounded value whatever the summation order.  Write-bandwidth bound.  A
// sparse correction (orka README, "How it works": the decode plus a sparse
// correction) is added to the float64 value entry by entry, in storage
// order, then a low-rank correction's terms U[r][j] V[j][c] in order of j
// (orka README, CLI: the correct command), before the one rounding.
//
// Residual ladders (per-stage widths) and stage scales (GLQ page, "Inference
// kernels": the inverse residual scale of the two-stage call) take the
// BITS = 0 instantiation: each stage's width is read at run time, each
// entry is multiplied by its stage scale in float64 (exact: 24 + 11
// significant bits), the products are added from stage 0 up with float64
// rounding and the sum is multiplied by the block scale in float64 -- a
// fixed order, so the fp16 result is reproducible bit for bit.
//
// k_dequant_lds serves the formats whose codebooks fit LDS (8- and 12-bit
// stages, the ladders the decode kernels take) with K % 32 == 0: a
// persistent grid stages the codebooks once per workgroup, each thread
// takes four consecutive groups of a row at a time (one 4-byte load of low
// bytes and one 2-byte load of nibbles per stage, the next four groups'
// loads in flight), gathers from LDS, and writes 64 contiguous bytes.  The
// arithmetic per group is the same float64 sequence as above, so both
// kernels give identical bits.
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
  int lr_rank;              // low-rank correction U V, 0 = none
  const uint16_t *lr_u;     // fp16 [N][lr_rank]
  const uint16_t *lr_v;     // fp16 [lr_rank][K]
};

// The low-rank terms of group g of row r added to its float64 values: for
// j = 0, 1, ... in order, wv[q] += U[r][j] V[j][8g + q] (the fp16 product
// is exact in float64, so a fused multiply-add rounds the same).
__device__ __forceinline__ void add_lowrank(const DequantArgs &a, int64_t r, int g, double (&wv)[8]) {
  const uint16_t *ur = a.lr_u + r * a.lr_rank;
  for (int j = 0; j < a.lr_rank; ++j) {
    const double u = (double)h2f(ur[j]);
    const uint4 h = *reinterpret_cast<const uint4 *>(a.lr_v + (int64_t)j * a.k + 8 * g);
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) wv[q] = wv[q] + u * (double)h2f((hw[q >> 1] >> (16 * (q & 1))) & 0xffffu);
  }
}

// The eight fp16 results of a group, two per word: one test for the group,
// the hardware rounding when all eight are finite and below 65504, else the
// integer rounding for all eight (both round the float64 value once, to
// nearest even).
__device__ __forceinline__ uint4 round_group_f16(const double (&wv)[8]) {
  bool easy = true;
#pragma unroll
  for (int j = 0; j < 8; ++j) easy = easy && __builtin_fabs(wv[j]) < 65504.0;
  uint32_t o[4];
  if (easy) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f64_to_f16_rn_odd(wv[2 * j]) | (f64_to_f16_rn_odd(wv[2 * j + 1]) << 16);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f64_to_f16_rne(wv[2 * j]) | (f64_to_f16_rne(wv[2 * j + 1]) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

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
  if (a.lr_rank > 0) add_lowrank(a, r, g, wv);
  reinterpret_cast<uint4 *>(a.w_out + r * (int64_t)a.k)[g] = round_group_f16(wv);
}

constexpr int kDqThreads = 1024;

// value of group f (row r, group g of the row) from its stage entries (c_t
// already gathered), in the float64 order of k_unpack_dequant, stored as 8
// fp16
template <int S, bool RS>
__device__ __forceinline__ void dequant_group(const DequantArgs &a, const uint4 (&v)[S], int64_t r, int g) {
  double acc[8];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const uint32_t h[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double c = (double)h2f((h[j >> 1] >> ((j & 1) * 16)) & 0xffffu);
      if (RS) c *= (double)a.rs[t];  // exact product
      acc[j] = (t == 0) ? c : acc[j] + c;
    }
  }
  const double sc = (double)h2f(a.sc[r * a.nblk + (8 * g) / a.bs]);
  double wv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wv[j] = sc * acc[j];
  if (a.sp_nnz > 0) {
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
      const double sv = (double)h2f(a.sp_val[j]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q == c) wv[q] = wv[q] + sv;
    }
  }
  if (a.lr_rank > 0) add_lowrank(a, r, g, wv);
  reinterpret_cast<uint4 *>(a.w_out + r * (int64_t)a.k)[g] = round_group_f16(wv);
}

template <class LD, bool RS>
__global__ __launch_bounds__(kDqThreads) void k_dequant_lds(DequantArgs a) {
  constexpr int S = LD::S;
  __shared__ uint4 s_cb[LD::kRows];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t quads = a.total / 4;  // G % 4 == 0: a quad never crosses a row
  const int64_t stride = (int64_t)gridDim.x * kDqThreads;
  struct QIdx {
    uint32_t lo[S];  // four low bytes
    uint32_t hi[S];  // four nibbles
  };
  auto load_q = [&](int64_t q, QIdx &I) {
    const int64_t f0 = 4 * (q < quads ? q : quads - 1);  // past the end: the last quad again
#pragma unroll
    for (int t = 0; t < S; ++t) {
      I.lo[t] = LD::lo(t) ? *reinterpret_cast<const uint32_t *>(a.lo[t] + f0) : 0u;
      I.hi[t] = LD::hi(t) ? *reinterpret_cast<const uint16_t *>(a.hi[t] + (f0 >> 1)) : 0u;
    }
  };
  int64_t q = (int64_t)blockIdx.x * kDqThreads + tid;
  QIdx cur;
  load_q(q, cur);
  if constexpr (LD::kUniform) {
    constexpr int BITS = LD::bits(0);
    constexpr int CBN = S << BITS;
    for (int blk = wave * 64; blk < CBN; blk += kDqThreads) {  // wave-uniform
      lds_direct_16(reinterpret_cast<const uint4 *>(uniform_ptr(a.cb[blk >> BITS])) + (blk & ((1 << BITS) - 1)) + lane,
                    s_cb + blk);
    }
  } else {
    stage_ladder_lds<LD, kDqThreads / 64>(a.cb, s_cb, wave, lane);
  }
  wait_all_memory();  // the codebooks (LDS-direct) have landed
  __syncthreads();
  for (; q < quads; q += stride) {
    QIdx nxt;
    load_q(q + stride, nxt);
    const int64_t f0 = 4 * q;
    const int64_t r = f0 / a.G;
    const int g0 = (int)(f0 - r * a.G);
    uint32_t id[S][4];
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        uint32_t idx = 0;
        if (LD::lo(t)) idx = (cur.lo[t] >> (8 * gg)) & 0xffu;
        if (LD::hi(t)) idx |= ((cur.hi[t] >> (4 * gg)) & 0xfu) << LD::hshift(t);
        id[t][gg] = idx;
      }
    if (a.idx_out) {
#pragma unroll
      for (int t = 0; t < S; ++t)
        *reinterpret_cast<uint2 *>(a.idx_out + (int64_t)t * a.total + f0) =
            make_uint2(id[t][0] | (id[t][1] << 16), id[t][2] | (id[t][3] << 16));
    }
    if (a.w_out) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        uint4 v[S];
#pragma unroll
        for (int t = 0; t < S; ++t) v[t] = s_cb[LD::off(t) + id[t][gg]];
        dequant_group<S, RS>(a, v, r, g0 + gg);
      }
    }
    cur = nxt;
  }
}

template <class LD, bool RS>
static void launch_dq(const DequantArgs &a, hipStream_t s) {
  const int64_t need = (a.total / 4 + kDqThreads - 1) / kDqThreads;
  const int cus = device_cu_count();
  const unsigned grid = (unsigned)(need < cus ? need : cus);
  hipLaunchKernelGGL((k_dequant_lds<LD, RS>), dim3(grid), dim3(kDqThreads), 0, s, a);
}

// the LDS kernel for this format, if it has one (false: nothing launched)
static bool launch_dequant_lds(const WView &w, const DequantArgs &a, hipStream_t s) {
  if (w.k % 32 != 0) return false;
  const int b0 = w.sb[0], b1 = w.S > 1 ? w.sb[1] : 0;
  if (w.uniform && !w.scaled) {
    if (w.bits == 12 && w.S == 1) return launch_dq<Ladder<12>, false>(a, s), true;
    if (w.bits == 12 && w.S == 2) return launch_dq<Ladder<12, 12>, false>(a, s), true;
    if (w.bits == 8 && w.S == 1) return launch_dq<Ladder<8>, false>(a, s), true;
    if (w.bits == 8 && w.S == 2) return launch_dq<Ladder<8, 8>, false>(a, s), true;
    if (w.bits == 8 && w.S == 3) return launch_dq<Ladder<8, 8, 8>, false>(a, s), true;
    if (w.bits == 8 && w.S == 4) return launch_dq<Ladder<8, 8, 8, 8>, false>(a, s), true;
    return false;
  }
  if (w.S > 2) return false;
  if (!w.scaled) {
    if (b0 == 12 && b1 == 4) return launch_dq<Ladder<12, 4>, false>(a, s), true;
    if (b0 == 8 && b1 == 4) return launch_dq<Ladder<8, 4>, false>(a, s), true;
    return false;
  }
  if (b0 == 12 && b1 == 0) return launch_dq<Ladder<12>, true>(a, s), true;
  if (b0 == 8 && b1 == 0) return launch_dq<Ladder<8>, true>(a, s), true;
  if (b0 == 12 && b1 == 12) return launch_dq<Ladder<12, 12>, true>(a, s), true;
  if (b0 == 8 && b1 == 8) return launch_dq<Ladder<8, 8>, true>(a, s), true;
  if (b0 == 12 && b1 == 4) return launch_dq<Ladder<12, 4>, true>(a, s), true;
  if (b0 == 8 && b1 == 4) return launch_dq<Ladder<8, 4>, true>(a, s), true;
  return false;
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
  a.lr_rank = w.lr_rank;
  a.lr_u = w.lr_u;
  a.lr_v = w.lr_v;
  if (launch_dequant_lds(w, a, s)) return hipGetLastError();
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
