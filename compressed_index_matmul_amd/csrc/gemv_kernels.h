// Kernel templates of the decode-path product y = x dequant(W)^T, shared by
// the translation units that instantiate them (k_gemv.hip: the plain
// formats; k_gemv_ladder.hip: mixed-width ladders and stage scales).
#pragma once

#include "vqmm_device.h"
#include "vqmm_internal.h"

namespace vqmm {

struct GemvArgs {
  const uint8_t *lo[VQ_MAX_STAGES];
  const uint8_t *hi[VQ_MAX_STAGES];
  const uint16_t *i16[VQ_MAX_STAGES];
  const uint16_t *cb[VQ_MAX_STAGES];
  const uint16_t *sc;
  const void *x;  // this token's row
  float *y;       // this token's row
  int n, k, G, S, nblk, bs;
  int C;          // 4-group chunks per row (G / 4) -- fast path
  int sb[VQ_MAX_STAGES];    // index width of each stage
  float rs[VQ_MAX_STAGES];  // stage scales (1 when the weight has none)
  int sp_nnz;               // sparse correction (CSR over rows), 0 = none
  const int32_t *sp_rowptr;
  const int32_t *sp_col;
  const uint16_t *sp_val;
};

// ---------------------------------------------------------------------------
// fast path
// ---------------------------------------------------------------------------
// LDS bytes of the fast kernel: codebooks, x (fp16: 64 B per 4-group chunk
// plus a float factor; fp32: 128 B per chunk) for 64 * CPL chunks.
__host__ __device__ constexpr size_t gemv_lds_bytes(int cb_rows, int CPL, bool XF16, int T = 1) {
  return (size_t)cb_rows * 16 + (size_t)T * (64 * CPL * (XF16 ? 64 + 4 : 128 + 0) + (XF16 ? 0 : 4));
}
constexpr size_t kLdsBytes = 163840;  // 160 KiB per workgroup on gfx950

// LD is the stage ladder (index widths, see Ladder); RS: stage t's partial
// dot product is multiplied by its stage scale a.rs[t]; SP: the weight has a
// sparse correction, added to each row's sum.
template <class LD, bool RS, int CPL, int WAVES, bool XF16, int D, bool XREG, bool PIPE, int T = 1, bool SP = false>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_lds(GemvArgs a) {
  constexpr int S = LD::S;
  constexpr int NT = WAVES * 64;
  constexpr int CBN = LD::kRows;                  // codebook rows of all stages
  constexpr int CB_ITERS = (CBN + NT - 1) / NT;  // 1 KiB LDS-direct loads per wave
  constexpr int XV = XF16 ? 4 : 8;               // 16-byte x vectors per chunk
  constexpr int CMAX = 64 * CPL;                 // chunk capacity
  constexpr int XCH = (CMAX + NT - 1) / NT;      // x chunks converted per thread
  static_assert(XF16 || XREG, "fp32 x is always held in registers");
  static_assert(T == 1 || (XF16 && XREG), "several tokens: bf16 x held in registers");
  // x in LDS is vector-major (s_x[v * CMAX + c]) so that a wave reading the
  // same vector of 64 consecutive chunks touches consecutive 16-byte slots.
  __shared__ uint4 s_cb[CBN];
  __shared__ uint4 s_x[T][CMAX * XV];  // T tokens (x is [T][k])
  __shared__ float s_f[T][XF16 ? CMAX : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: row math stays scalar
  // Each workgroup owns a contiguous block of rows (equal sizes up to one
  // row); its waves take every WAVES-th row of the block.
  const int per_wg = (a.n + gridDim.x - 1) / gridDim.x;
  const int blk_lo = blockIdx.x * per_wg;
  const int blk_hi = min(a.n, blk_lo + per_wg);
  constexpr int stride = WAVES;
  const int row0 = blk_lo + wave;
  const int last = a.n - 1;
  const int nrows = row0 < blk_hi ? (blk_hi - 1 - row0) / stride + 1 : 0;  // rows of this wave (uniform)

  // This lane's chunks and their byte offsets within a row of each plane
  // (low bytes: 4 per chunk; high nibbles: 2 per chunk; scales: the chunk's
  // scale block).  Chunks past the end of the row reuse the last chunk.
  int cc[CPL];
  bool ok[CPL];
  uint32_t vlo[CPL], vsc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    ok[j] = c < a.C;
    cc[j] = ok[j] ? c : a.C - 1;
    vlo[j] = 4u * cc[j];
    vsc[j] = 2u * (uint32_t)((32 * cc[j]) / a.bs);
  }
  // Buffer descriptors: a load is descriptor + lane offset + a wave-uniform
  // row offset held in a scalar register, so no per-lane 64-bit address
  // arithmetic.  Every plane is below 2^31 bytes (n_out * k_in < 2^31).
  const uint32_t plane = (uint32_t)a.n * (uint32_t)a.G;
  buf_t blo[S], bhi[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    blo[t] = make_buf(LD::lo(t) ? a.lo[t] : a.hi[t], plane);
    bhi[t] = make_buf(LD::hi(t) ? a.hi[t] : a.lo[t], (plane + 1) / 2);
  }
  const buf_t bsc = make_buf(a.sc, 2u * (uint32_t)a.n * (uint32_t)a.nblk);
  // Sparse correction (orka README, "How it works": the decode plus a sparse
  // correction): lane i holds the CSR range of the wave's row i (rows < 64),
  // loaded before everything else; a row's first kSpRing entries travel in
  // the row ring with its index planes, kSpPer per lane.  Descriptors of zero
  // size without a correction.
  constexpr int kSpPer = SP ? 1 : 0;
  constexpr int kSpRing = 64 * kSpPer;
  const bool sp = SP && a.sp_nnz > 0;  // wave-uniform
  const buf_t bsp_ptr = make_buf(a.sp_rowptr, sp ? 4u * ((uint32_t)a.n + 1u) : 0u);
  const buf_t bsp_col = make_buf(a.sp_col, sp ? 4u * (uint32_t)a.sp_nnz : 0u);
  const buf_t bsp_val = make_buf(a.sp_val, sp ? 2u * (uint32_t)a.sp_nnz : 0u);
  uint32_t sp_lo = 0, sp_hi = 0;
  if (sp) {
    const uint32_t ri = (uint32_t)min(row0 + min(lane, max(nrows - 1, 0)) * stride, last);
    sp_lo = buf_u32(bsp_ptr, 4u * ri, 0);
    sp_hi = buf_u32(bsp_ptr, 4u * ri + 4u, 0);
  }
  sched_fence();
  // CSR range of the wave's row r (wave-uniform), clamped to the arrays
  auto sp_range = [&](int r, int &lo, int &hi) {
    if (r < 64) {
      lo = __builtin_amdgcn_readlane((int)sp_lo, r);
      hi = __builtin_amdgcn_readlane((int)sp_hi, r);
    } else {
      const int rr = min(row0 + r * stride, last);
      lo = a.sp_rowptr[rr];
      hi = a.sp_rowptr[rr + 1];
    }
    lo = min(max(lo, 0), a.sp_nnz);
    hi = min(max(hi, lo), a.sp_nnz);
  };

  // Index planes and scales of one row (this lane's chunks), and this lane's
  // entry of the row's sparse correction.
  struct RowIdx {
    uint32_t L[CPL][S];
    uint32_t H[CPL][S];
    uint32_t SC[CPL];
    uint32_t SPC[kSpPer], SPV[kSpPer];
  };
  auto load_row = [&](int r, RowIdx &R) {
    // past the wave's last row: that row again (an L2 hit, never stored)
    const uint32_t rr = (uint32_t)min(row0 + min(r, nrows - 1) * stride, last);
    const uint32_t rb = rr * (uint32_t)a.G;  // G is a multiple of 4 here
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
#pragma unroll
      for (int t = 0; t < S; ++t) {
        if (LD::lo(t)) R.L[j][t] = buf_u32(blo[t], vlo[j], rb);
        if (LD::hi(t)) R.H[j][t] = buf_u16(bhi[t], vlo[j] >> 1, rb >> 1);
      }
      R.SC[j] = buf_u16(bsc, vsc[j], 2u * rr * (uint32_t)a.nblk);
    }
    if (sp) {
      sched_fence();  // the index loads go out before the wait on the CSR range
      int lo, hi;
      sp_range(max(min(r, nrows - 1), 0), lo, hi);
      // every load is issued by every lane (a clamped duplicate past the
      // row's entries): the prologue's wait counts them
#pragma unroll
      for (int e = 0; e < kSpPer; ++e) {
        const uint32_t j = (uint32_t)min(lo + 64 * e + lane, max(hi - 1, 0));
        R.SPC[e] = buf_u32(bsp_col, 4u * j, 0);
        R.SPV[e] = buf_u16(bsp_val, 2u * j, 0);
      }
    }
  };

  // Global loads are issued in the order they are needed: the codebooks
  // straight into LDS (global_load_lds_dwordx4: lane l of a wave writes 16
  // bytes at the wave's LDS base + 16 l), this thread's x chunks, then the
  // first D rows' index planes from HBM.  Loads complete in issue order, so
  // once at most the index loads are outstanding the codebooks and x have
  // landed; the HBM latency of the index loads then overlaps the x
  // conversion and the barrier.  No branch surrounds an index load:
  // out-of-range chunks and rows load a valid duplicate and are discarded.
  if constexpr (LD::kBlocks && LD::kUniform) {
#pragma unroll
    for (int r = 0; r < CB_ITERS; ++r) {
      const int blk = (r * WAVES + wave) * 64;  // first codebook row of this wave's 1 KiB
      if (blk < CBN) {
        // a whole block of one stage (wave-uniform stage)
        constexpr int B = LD::bits(0);
        const uint4 *src = reinterpret_cast<const uint4 *>(a.cb[blk >> B]) + (blk & ((1 << B) - 1)) + lane;
        lds_direct_16(src, s_cb + blk);
      }
    }
  } else {
    stage_ladder_lds<LD, WAVES>(a.cb, s_cb, wave, lane);  // mixed widths
  }
  sched_fence();
  // (waves whose x chunks all lie past the end of x load none: a
  // wave-uniform branch)
  uint4 xin[T][XCH][XV];
  const uint32_t xrow = (uint32_t)a.k * (XF16 ? 2u : 4u);  // bytes per token
  const buf_t bx = make_buf(a.x, xrow * T);
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      if (wave * 64 + NT * i < a.C) {
        const uint32_t c = (uint32_t)min(tid + NT * i, a.C - 1);
#pragma unroll
        for (int v = 0; v < XV; ++v) xin[tt][i][v] = buf_u128(bx, c * (16u * XV) + 16u * v, xrow * tt);
      }
    }
  sched_fence();
  RowIdx R[D + 1];
#pragma unroll
  for (int k = 0; k < D; ++k) load_row(k, R[k]);
  sched_fence();
  constexpr int kIdxLoads = D * CPL * (LD::kPlanes + 1);
  constexpr int kSpLoads = kIdxLoads + 2 * kSpPer * D;  // with a correction: + columns and values
  if (sp) wait_vmem<(kSpLoads < 63 ? kSpLoads : 63)>();
  else wait_vmem<(kIdxLoads < 63 ? kIdxLoads : 63)>();

  // x -> LDS.  bf16 x becomes fp16 after a per-chunk power-of-two rescale
  // that puts the chunk's largest |x| in [2^14, 2^15): exact for every value
  // within 2^28 of that maximum.  The chunk's partial dot product is scaled
  // back by s_f[c].
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tid + NT * i;
    if (c < a.C) {
      if (XF16) {
        float mx = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t w4[4] = {xin[tt][i][v].x, xin[tt][i][v].y, xin[tt][i][v].z, xin[tt][i][v].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mx = fmaxf(mx, fmaxf(fabsf(bf2f(w4[e] & 0xffffu)), fabsf(bf2f(w4[e] >> 16))));
        }
        const int xexp = (mx > 0.f && mx <= 3.0e38f) ? 14 - ilogbf(mx) : 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t w4[4] = {xin[tt][i][v].x, xin[tt][i][v].y, xin[tt][i][v].z, xin[tt][i][v].w};
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const half2_t h = half2_t{(_Float16)ldexpf(bf2f(w4[e] & 0xffffu), xexp),
                                      (_Float16)ldexpf(bf2f(w4[e] >> 16), xexp)};
            o[e] = __builtin_bit_cast(uint32_t, h);
          }
          s_x[tt][v * CMAX + c] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        s_f[tt][c] = ldexpf(1.f, -xexp);
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) s_x[tt][v * CMAX + c] = xin[tt][i][v];
      }
    }
  }
  // this wave's codebook part landed before its x; the barrier makes every
  // wave's codebook part and x visible, with the first rows' index loads
  // still in flight (lds_barrier, not __syncthreads: that would wait for them)
  lds_barrier();

  // this lane's x chunks: registers for the whole launch (XREG) or LDS reads
  // per use; the per-chunk factor, zero for chunks past the end of the row
  half2_t xh[T][XREG && XF16 ? CPL : 1][16];
  float xf[XF16 ? 1 : CPL][32];
  float fm[T][CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      fm[tt][j] = XF16 ? (ok[j] ? s_f[tt][cc[j]] : 0.f) : (ok[j] ? 1.f : 0.f);
      if (XF16 && XREG) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 u = s_x[tt][v * CMAX + cc[j]];
          xh[tt][j][4 * v + 0] = as_h2(u.x);
          xh[tt][j][4 * v + 1] = as_h2(u.y);
          xh[tt][j][4 * v + 2] = as_h2(u.z);
          xh[tt][j][4 * v + 3] = as_h2(u.w);
        }
      }
    }
    if (!XF16) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const uint4 u = s_x[0][v * CMAX + cc[j]];
        xf[j][4 * v + 0] = __uint_as_float(u.x);
        xf[j][4 * v + 1] = __uint_as_float(u.y);
        xf[j][4 * v + 2] = __uint_as_float(u.z);
        xf[j][4 * v + 3] = __uint_as_float(u.w);
      }
    }
  }

  // One item = one 4-group chunk of a row: S x 4 LDS gathers (in the order
  // the dot products consume them) and, without XREG, the chunk's 64 B of x.
  struct Item {
    uint4 v[S][4];
    uint4 x[XREG ? 1 : 4];
  };
  auto gather = [&](const RowIdx &Rr, int j, Item &it) {
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t idx = 0;
        if (LD::lo(t)) idx = (Rr.L[j][t] >> (8 * q)) & 0xffu;
        if (LD::hi(t)) idx |= ((Rr.H[j][t] >> (4 * q)) & 0xfu) << LD::hshift(t);
        it.v[t][q] = s_cb[LD::off(t) + idx];
      }
    if (!XREG) {
#pragma unroll
      for (int v = 0; v < 4; ++v) it.x[v] = s_x[0][v * CMAX + cc[j]];
    }
  };
  // dot products of chunk j's gathered vectors with x of every token (with
  // RS each stage's partial is formed on its own and then scaled)
  auto dot = [&](int j, const Item &it, float (&d)[T]) {
#pragma unroll
    for (int tt = 0; tt < T; ++tt) d[tt] = 0.f;
#pragma unroll
    for (int t = 0; t < S; ++t) {
      float e[T];
#pragma unroll
      for (int tt = 0; tt < T; ++tt) e[tt] = RS ? 0.f : d[tt];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (XF16) {
#pragma unroll
          for (int tt = 0; tt < T; ++tt) {
            const uint4 xq = it.x[XREG ? 0 : q];
            const half2_t x0 = XREG ? xh[tt][XREG ? j : 0][4 * q + 0] : as_h2(xq.x);
            const half2_t x1 = XREG ? xh[tt][XREG ? j : 0][4 * q + 1] : as_h2(xq.y);
            const half2_t x2 = XREG ? xh[tt][XREG ? j : 0][4 * q + 2] : as_h2(xq.z);
            const half2_t x3 = XREG ? xh[tt][XREG ? j : 0][4 * q + 3] : as_h2(xq.w);
            e[tt] = __builtin_amdgcn_fdot2(as_h2(it.v[t][q].x), x0, e[tt], false);
            e[tt] = __builtin_amdgcn_fdot2(as_h2(it.v[t][q].y), x1, e[tt], false);
            e[tt] = __builtin_amdgcn_fdot2(as_h2(it.v[t][q].z), x2, e[tt], false);
            e[tt] = __builtin_amdgcn_fdot2(as_h2(it.v[t][q].w), x3, e[tt], false);
          }
        } else {
          const uint32_t hv[4] = {it.v[t][q].x, it.v[t][q].y, it.v[t][q].z, it.v[t][q].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            e[0] = fmaf(h2f(hv[c] & 0xffffu), xf[XF16 ? 0 : j][8 * q + 2 * c], e[0]);
            e[0] = fmaf(h2f(hv[c] >> 16), xf[XF16 ? 0 : j][8 * q + 2 * c + 1], e[0]);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < T; ++tt) d[tt] = !RS ? e[tt] : t == 0 ? e[tt] * a.rs[0] : fmaf(a.rs[t], e[tt], d[tt]);
    }
  };
  // One row: CPL items (with PIPE the gathers of chunk j+1 are issued before
  // the dot products of chunk j), one fixed-order wave reduction.
  auto compute_row = [&](int r, const RowIdx &Rr) {
    float acc[T];
    auto add = [&](int j, const Item &it) {
      float d[T];
      dot(j, it, d);
      const float sc = h2f(Rr.SC[j]);
#pragma unroll
      for (int tt = 0; tt < T; ++tt) {
        const float f = sc * fm[tt][j];
        acc[tt] = j == 0 ? f * d[tt] : fmaf(f, d[tt], acc[tt]);
      }
    };
    if (PIPE) {
      Item ia, ib;
      gather(Rr, 0, ia);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        sched_fence();
        if (j + 1 < CPL) gather(Rr, j + 1, (j & 1) ? ia : ib);
        sched_fence();
        add(j, (j & 1) ? ib : ia);
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        Item it;
        gather(Rr, j, it);
        add(j, it);
      }
    }
    if (sp) {
      // x of column c, token tt, from the staged copy
      auto x_at = [&](int tt, int c) -> float {
        const int ch = c >> 5, p = c & 31;
        if (XF16) {
          const _Float16 *hx = reinterpret_cast<const _Float16 *>(&s_x[tt][(p >> 3) * CMAX + ch]);
          return (float)hx[p & 7] * s_f[tt][ch];
        }
        const float *fx = reinterpret_cast<const float *>(&s_x[0][(p >> 2) * CMAX + ch]);
        return fx[p & 3];
      };
      int lo, hi;
      sp_range(r, lo, hi);
      // the first kSpRing entries come from the ring, any further ones are
      // loaded here
#pragma unroll
      for (int e = 0; e < kSpPer; ++e) {
        const bool has = lo + 64 * e + lane < hi;
        const int c = (int)Rr.SPC[e];
        if (has && c >= 0 && c < a.k) {
          const float v = h2f(Rr.SPV[e]);
#pragma unroll
          for (int tt = 0; tt < T; ++tt) acc[tt] = fmaf(v, x_at(tt, c), acc[tt]);
        }
      }
      for (int j0 = lo + kSpRing; j0 < hi; j0 += 64) {
        const bool has = j0 + lane < hi;
        const int c = has ? a.sp_col[j0 + lane] : -1;
        if (c >= 0 && c < a.k) {
          const float v = h2f(a.sp_val[j0 + lane]);
#pragma unroll
          for (int tt = 0; tt < T; ++tt) acc[tt] = fmaf(v, x_at(tt, c), acc[tt]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const float tot = wave_sum(acc[tt]);
      if (lane == 0) a.y[(size_t)tt * a.n + row0 + r * stride] = tot;
    }
  };

  // Ring of D+1 row buffers: row r+D's index loads are issued before row r is
  // computed, so D rows of HBM loads stay in flight per wave.
  int r = 0;
  for (; r + (D + 1) <= nrows; r += D + 1) {
#pragma unroll
    for (int k = 0; k <= D; ++k) {
      load_row(r + k + D, R[(k + D) % (D + 1)]);
      sched_fence();
      compute_row(r + k, R[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < D; ++k)
    if (r + k < nrows) compute_row(r + k, R[k]);
}

// ---------------------------------------------------------------------------
// general path
// ---------------------------------------------------------------------------
constexpr int kGenWaves = 8;
constexpr int kGenMaxXLds = 32768;  // fp32 x elements staged in LDS (128 KiB)

// BITS: the index width of every stage, or 0 for a ladder of per-stage
// widths (a.sb) whose stage partials are multiplied by the stage scales.
template <int BITS, int GPL, bool X_LDS>
__global__ __launch_bounds__(kGenWaves * 64) void k_gemv_gen(GemvArgs a, int xt) {
  __shared__ float s_x[X_LDS ? kGenMaxXLds : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  if (X_LDS) {
    for (int i = tid; i < a.k; i += kGenWaves * 64) {
      s_x[i] = (xt == VQ_F32) ? reinterpret_cast<const float *>(a.x)[i]
                              : bf2f(reinterpret_cast<const uint16_t *>(a.x)[i]);
    }
    __syncthreads();
  }
  const int units = a.G / GPL;  // lane work units per row
  for (int row = blockIdx.x * kGenWaves + wave; row < a.n; row += gridDim.x * kGenWaves) {
    const size_t rb = (size_t)row * a.G;
    float acc = 0.f;
    for (int u = lane; u < units; u += 64) {
      const int g0 = u * GPL;
      float d[GPL];
#pragma unroll
      for (int q = 0; q < GPL; ++q) d[q] = 0.f;
      for (int t = 0; t < a.S; ++t) {
        const int bt = BITS ? BITS : a.sb[t];  // wave-uniform
        uint32_t idx[GPL];
        if constexpr (GPL == 4) {
          if (bt == 16) {
            const uint2 v = *reinterpret_cast<const uint2 *>(a.i16[t] + rb + g0);
            idx[0] = v.x & 0xffffu;
            idx[1] = v.x >> 16;
            idx[2] = v.y & 0xffffu;
            idx[3] = v.y >> 16;
          } else {
            const uint32_t lw = bt == 4 ? 0u : *reinterpret_cast<const uint32_t *>(a.lo[t] + rb + g0);
            uint32_t hw = 0;
            if (bt == 12 || bt == 4) hw = *reinterpret_cast<const uint16_t *>(a.hi[t] + ((rb + g0) >> 1));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t nib = (hw >> (4 * q)) & 0xfu;
              idx[q] = bt == 4 ? nib : ((lw >> (8 * q)) & 0xffu) | (bt == 12 ? nib << 8 : 0u);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < GPL; ++q) idx[q] = load_index(bt, a.lo[t], a.hi[t], a.i16[t], rb + g0 + q);
        }
        uint4 cv[GPL];
#pragma unroll
        for (int q = 0; q < GPL; ++q) cv[q] = reinterpret_cast<const uint4 *>(a.cb[t])[idx[q]];
#pragma unroll
        for (int q = 0; q < GPL; ++q) {
          const uint32_t hv[4] = {cv[q].x, cv[q].y, cv[q].z, cv[q].w};
          const int col = 8 * (g0 + q);
          float xv[8];
          if (X_LDS) {
            const float4 x0 = *reinterpret_cast<const float4 *>(&s_x[col]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&s_x[col + 4]);
            xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w;
            xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              xv[e] = (xt == VQ_F32) ? reinterpret_cast<const float *>(a.x)[col + e]
                                     : bf2f(reinterpret_cast<const uint16_t *>(a.x)[col + e]);
          }
          float p = BITS ? d[q] : 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p = fmaf(h2f(hv[e] & 0xffffu), xv[2 * e], p);
            p = fmaf(h2f(hv[e] >> 16), xv[2 * e + 1], p);
          }
          d[q] = BITS ? p : fmaf(a.rs[t], p, d[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < GPL; ++q) {
        const float s = h2f(a.sc[(size_t)row * a.nblk + (8 * (g0 + q)) / a.bs]);
        acc = fmaf(s, d[q], acc);
      }
    }
    const float tot = wave_sum(acc);
    if (lane == 0) a.y[row] = tot;
  }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
static GemvArgs make_args(const WView &w) {
  GemvArgs a{};
  for (int t = 0; t < VQ_MAX_STAGES; ++t) {
    a.lo[t] = w.lo[t];
    a.hi[t] = w.hi[t];
    a.i16[t] = w.i16[t];
    a.cb[t] = w.cb[t];
  }
  a.sc = w.sc;
  a.n = w.n;
  a.k = w.k;
  a.G = w.G;
  a.S = w.S;
  a.nblk = w.nblk;
  a.bs = w.bs;
  a.C = w.G / 4;
  for (int t = 0; t < VQ_MAX_STAGES; ++t) {
    a.sb[t] = t < w.S ? w.sb[t] : 0;
    a.rs[t] = w.rs[t];
  }
  a.sp_nnz = w.sp_nnz;
  a.sp_rowptr = w.sp_rowptr;
  a.sp_col = w.sp_col;
  a.sp_val = w.sp_val;
  return a;
}

template <class LD, bool RS, int CPL, int W, int D, bool XF16, bool XREG, bool PIPE, bool SP>
static void launch_fast_w(const GemvArgs &a, int cus, hipStream_t s) {
  const int g = (a.n + W - 1) / W;
  hipLaunchKernelGGL((k_gemv_lds<LD, RS, CPL, W, XF16, D, XREG, PIPE, 1, SP>), dim3(g < cus ? g : cus), dim3(W * 64),
                     0, s, a);
}

// Persistent grid of one workgroup per CU (the codebooks and x take most of
// the LDS).  Waves per workgroup, the prefetch depth D (rows of index loads
// in flight per wave) and in-row gather pipelining trade registers: 16 waves
// get 128 VGPRs each, 8 get 256.  Rows of 1-2 chunks per lane: 16 waves, x in
// registers; 3-4 chunks: 8 waves, two rows in flight, pipelined gathers;
// longer rows: 8 waves, x read from LDS per chunk.
template <class LD, bool RS, int CPL, bool XF16, bool SP>
static void launch_fast_c(const GemvArgs &a, int cus, hipStream_t s) {
  if constexpr (gemv_lds_bytes(LD::kRows, CPL, XF16) <= kLdsBytes) {
    if constexpr (CPL <= 2) launch_fast_w<LD, RS, CPL, 16, 1, XF16, true, false, SP>(a, cus, s);
    else if constexpr (CPL <= 4 || !XF16) launch_fast_w<LD, RS, CPL, 8, 2, XF16, true, true, SP>(a, cus, s);
    else launch_fast_w<LD, RS, CPL, 8, 1, XF16, false, true, SP>(a, cus, s);
  }
}

// One token through the LDS kernel of ladder LD (the caller has checked
// gemv_fast_shape).
template <class LD, bool RS, bool XF16, bool SP = false>
static void launch_fast_s(const GemvArgs &a, int cus, hipStream_t s) {
  switch ((a.C + 63) / 64) {
    case 1: launch_fast_c<LD, RS, 1, XF16, SP>(a, cus, s); break;
    case 2: launch_fast_c<LD, RS, 2, XF16, SP>(a, cus, s); break;
    case 3: launch_fast_c<LD, RS, 3, XF16, SP>(a, cus, s); break;
    case 4: launch_fast_c<LD, RS, 4, XF16, SP>(a, cus, s); break;
    case 5: if constexpr (XF16) launch_fast_c<LD, RS, 5, XF16, SP>(a, cus, s); break;
    case 6: if constexpr (XF16) launch_fast_c<LD, RS, 6, XF16, SP>(a, cus, s); break;
    case 7: if constexpr (XF16) launch_fast_c<LD, RS, 7, XF16, SP>(a, cus, s); break;
    default: if constexpr (XF16) launch_fast_c<LD, RS, 8, XF16, SP>(a, cus, s); break;
  }
}

// 2..4 bf16 tokens in one launch of the LDS kernel: every gathered codebook
// vector is multiplied with the x of all tokens (held in registers), so the
// gathers, the LDS-bound part, are shared.  Rows of up to 3 chunks per lane
// (K <= 6144), at most 6 chunks x tokens, codebooks and all tokens' x in the
// LDS; other shapes take the matrix-core path.
template <class LD, bool RS, int CPL, int T, bool SP>
static bool launch_tokens_c(const GemvArgs &a, int cus, hipStream_t s) {
  // chunks x tokens <= 6 keeps x in registers without spills at 256 VGPRs
  if constexpr (CPL * T <= 6 && gemv_lds_bytes(LD::kRows, CPL, true, T) <= kLdsBytes) {
    const int g = (a.n + 7) / 8;
    hipLaunchKernelGGL((k_gemv_lds<LD, RS, CPL, 8, true, 1, true, false, T, SP>), dim3(g < cus ? g : cus), dim3(512),
                       0, s, a);
    return true;
  }
  return false;
}

template <class LD, bool RS, int T, bool SP>
static bool launch_tokens_t(const GemvArgs &a, int cus, hipStream_t s) {
  switch ((a.C + 63) / 64) {
    case 1: return launch_tokens_c<LD, RS, 1, T, SP>(a, cus, s);
    case 2: return launch_tokens_c<LD, RS, 2, T, SP>(a, cus, s);
    case 3: return launch_tokens_c<LD, RS, 3, T, SP>(a, cus, s);
    default: return false;
  }
}

// 2..4 bf16 tokens through the LDS kernel of ladder LD; false when the shape
// does not fit it (nothing launched).
template <class LD, bool RS, bool SP = false>
static bool launch_tokens_s(const GemvArgs &a, int batch, int cus, hipStream_t s) {
  switch (batch) {
    case 2: return launch_tokens_t<LD, RS, 2, SP>(a, cus, s);
    case 3: return launch_tokens_t<LD, RS, 3, SP>(a, cus, s);
    case 4: return launch_tokens_t<LD, RS, 4, SP>(a, cus, s);
    default: return false;
  }
}

// ---------------------------------------------------------------------------
// format dispatch (templates on SP: each translation unit instantiates its
// share -- k_gemv.hip plain formats, k_gemv_ladder.hip ladders, both without
// a correction; k_gemv_sparse.hip both with one)
// ---------------------------------------------------------------------------
// Plain formats with an LDS kernel: 1-2 stages of 12 bits, 1-4 of 8 bits.
inline bool plain_lds_format(const WView &w) {
  return plain_format(w) && (w.bits == 8 || (w.bits == 12 && w.S <= 2));
}

template <bool SP, bool XF16>
static void launch_lds_plain(const WView &w, const GemvArgs &a, int cus, hipStream_t s) {
  if (w.bits == 12) {
    if (w.S == 1) launch_fast_s<Ladder<12>, false, XF16, SP>(a, cus, s);
    else launch_fast_s<Ladder<12, 12>, false, XF16, SP>(a, cus, s);
  } else {
    switch (w.S) {
      case 1: launch_fast_s<Ladder<8>, false, XF16, SP>(a, cus, s); break;
      case 2: launch_fast_s<Ladder<8, 8>, false, XF16, SP>(a, cus, s); break;
      case 3: launch_fast_s<Ladder<8, 8, 8>, false, XF16, SP>(a, cus, s); break;
      default: launch_fast_s<Ladder<8, 8, 8, 8>, false, XF16, SP>(a, cus, s); break;
    }
  }
}

template <bool SP>
static bool launch_tokens_plain(const WView &w, const GemvArgs &a, int batch, int cus, hipStream_t s) {
  if (w.bits == 12) {
    if (w.S == 1) return launch_tokens_s<Ladder<12>, false, SP>(a, batch, cus, s);
    if (w.S == 2) return launch_tokens_s<Ladder<12, 12>, false, SP>(a, batch, cus, s);
    return false;
  }
  switch (w.S) {
    case 1: return launch_tokens_s<Ladder<8>, false, SP>(a, batch, cus, s);
    case 2: return launch_tokens_s<Ladder<8, 8>, false, SP>(a, batch, cus, s);
    default: return false;
  }
}

// Ladders with an LDS kernel of their own: 12 + 4 and 8 + 4 bits (orka
// README quick start, the rvq-12-4 mode), and 1-2 stages of 8 or 12 bits
// with a residual scale per stage (GLQ page, "Inference kernels").
constexpr int ladder_pack2(int b0, int b1) { return (b0 / 4) | ((b1 / 4) << 4); }
inline int ladder_code2(const WView &w) { return w.S > 2 ? -1 : ladder_pack2(w.sb[0], w.S > 1 ? w.sb[1] : 0); }

template <bool SP, bool XF16>
static bool launch_lds_ladder(const WView &w, const GemvArgs &a, int cus, hipStream_t s) {
  const int code = ladder_code2(w);
  if (!w.scaled) {
    switch (code) {
      case ladder_pack2(12, 4): launch_fast_s<Ladder<12, 4>, false, XF16, SP>(a, cus, s); return true;
      case ladder_pack2(8, 4): launch_fast_s<Ladder<8, 4>, false, XF16, SP>(a, cus, s); return true;
      default: return false;
    }
  }
  switch (code) {
    case ladder_pack2(12, 0): launch_fast_s<Ladder<12>, true, XF16, SP>(a, cus, s); return true;
    case ladder_pack2(8, 0): launch_fast_s<Ladder<8>, true, XF16, SP>(a, cus, s); return true;
    case ladder_pack2(12, 12): launch_fast_s<Ladder<12, 12>, true, XF16, SP>(a, cus, s); return true;
    case ladder_pack2(8, 8): launch_fast_s<Ladder<8, 8>, true, XF16, SP>(a, cus, s); return true;
    case ladder_pack2(12, 4): launch_fast_s<Ladder<12, 4>, true, XF16, SP>(a, cus, s); return true;
    case ladder_pack2(8, 4): launch_fast_s<Ladder<8, 4>, true, XF16, SP>(a, cus, s); return true;
    default: return false;
  }
}

template <bool SP>
static bool launch_tokens_ladder(const WView &w, const GemvArgs &a, int batch, int cus, hipStream_t s) {
  const int code = ladder_code2(w);
  if (!w.scaled) {
    switch (code) {
      case ladder_pack2(12, 4): return launch_tokens_s<Ladder<12, 4>, false, SP>(a, batch, cus, s);
      case ladder_pack2(8, 4): return launch_tokens_s<Ladder<8, 4>, false, SP>(a, batch, cus, s);
      default: return false;
    }
  }
  switch (code) {
    case ladder_pack2(12, 12): return launch_tokens_s<Ladder<12, 12>, true, SP>(a, batch, cus, s);
    case ladder_pack2(12, 4): return launch_tokens_s<Ladder<12, 4>, true, SP>(a, batch, cus, s);
    default: return false;
  }
}

// Defined in k_gemv_ladder.hip (ladders, no correction) and k_gemv_sparse.hip
// (plain formats and ladders with a correction): false when the format has
// no LDS kernel (nothing launched).  The shape checks have been made.
bool launch_gemv_lds_ladder(const WView &w, const GemvArgs &a, bool xf16, int cus, hipStream_t s);
bool launch_gemv_tokens_ladder(const WView &w, const GemvArgs &a, int batch, int cus, hipStream_t s);
bool launch_gemv_lds_sparse(const WView &w, const GemvArgs &a, bool xf16, int cus, hipStream_t s);
bool launch_gemv_tokens_sparse(const WView &w, const GemvArgs &a, int batch, int cus, hipStream_t s);
// One stage of 16-bit indices (k_gemv_l2.hip): L2 gathers with the next
// row's indices loading and 16 gathers per lane in flight; false when the
// shape is not taken.
// The 16-bit decode kernel (k_gemv_l2.hip): whether it takes the weight, and
// its launch (false: nothing launched); signs (null: none) and max_block
// give the input transform it applies to x first.
bool gemv_l2_takes(const WView &w);
// One 16-bit stage with one scale per row, the codebook streamed through LDS
// in slices (k_gemv_cbs.hip): whether it takes the weight, and its launch for
// one token (false: nothing launched).
// With signs (max_block its largest block) the kernel applies the input
// transform to its own copy of x first; gemv_cbs_rht_takes says whether it
// can for this weight.
bool gemv_cbs_takes(const WView &w);
bool gemv_cbs_rht_takes(const WView &w);
bool launch_gemv_cbs(const WView &w, const void *x, int xt, float *y, int cus, hipStream_t s,
                     const int8_t *signs = nullptr, int max_block = 0);
bool launch_gemv_l2(const WView &w, const GemvArgs &a, int xt, int cus, hipStream_t s, const int8_t *signs = nullptr,
                    int max_block = 0);

}  // namespace vqmm
