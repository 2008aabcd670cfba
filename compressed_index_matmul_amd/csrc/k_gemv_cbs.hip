// Decode-path product for one stage of 16-bit indices into a 65,536-entry
// codebook (1 MiB; GLQ page, "How it works" / "Bit widths"), with the
// codebook streamed through LDS in slices instead of gathered from L2.
//
// The GLQ page ("Matched 4-bit head-to-head") names the gather of codebook
// vectors from the L2-cached codebook as what bounds its 4-bit kernel.  On
// gfx950 that gather is one L2 request per 8 weights, and the L2 serves
// about 12 of them per clock per XCD (counters: one request per gather, 98 %
// hits), which sets a floor of ~120 us for a 28672 x 8192 weight.  This
// kernel takes the gathers off the L2:
//   * every lane keeps, for the whole launch, the 16-bit indices of its
//     share of its rows in registers (read from HBM once), and its x columns
//     as fp16 (bf16 x is exact after a power-of-two rescale per lane; fp32 x,
//     e.g. after the input transform, is rounded to fp16);
//   * the codebook passes through LDS in P slices of S entries (one
//     workgroup per CU, the slice fills the LDS); in pass p a lane turns
//     each index into the byte offset (idx - p S) * 16, clamped from above
//     to the offset of one all-zero entry kept after the slice, so an index
//     outside the slice reads zeros and its dot product adds nothing.  Two
//     VALU instructions per index and pass (v_mad_u32_u16, v_min_u32) plus
//     the 16-byte LDS read and four v_dot2_f32_f16;
//   * indices outside the slice read the same zero entry (an LDS broadcast),
//     so a pass costs little more LDS time than its one in-slice gather per
//     index and P;
//   * per row the lane's products are summed in a fixed order (passes, then
//     slots), times the lane's rescale factor, reduced across the wave in a
//     fixed order, and the K parts of a row are added in a fixed order.  No
//     atomics; results do not depend on timing.
// Work split: a K part is 64 lanes x U index pairs (1024 U columns); lane l
// of K part q holds pairs q 64 U + l + 64 j, j < U (columns 16 pair ..
// 16 pair + 16).  K / (1024 U) K parts and 8 / that many row sets make up
// the 8 waves; a wave holds up to ROWS rows (ROWS x U index registers).
// Taken for one 16-bit stage, or a 16-bit stage plus a residual stage of
// 8-bit indices (its 4 KiB codebook in LDS beside the slice, one more pass
// after the slices; RES) or of 16-bit indices (its codebook streamed through
// the slices after the first's; ST2), stage scales allowed, one scale per row,
// K % 1024 == 0 with K / 1024 = U times 1, 2, 4 or 8.
#include <type_traits>

#include "gemv_kernels.h"

namespace vqmm {

namespace {

constexpr int kCbsWaves = 8;
constexpr int kCbsMaxSlice = 9408;  // entries per LDS slice: 147 KiB, a multiple of 64
constexpr int kCbsPasses = (65536 + kCbsMaxSlice - 1) / kCbsMaxSlice;  // 7

struct CbsArgs {
  const uint16_t *idx;  // 16-bit indices [n][G]
  const uint16_t *cb;   // fp16 [65536][8]
  const uint16_t *sc;   // fp16 per-row scales [n]
  const void *x;        // this token's row
  float *y;             // this token's row
  int xt;               // VQ_F32 / VQ_BF16
  int n, k, G;
  int kp;               // K parts (8 / row sets)
  int per_wg;           // rows per workgroup
  int slice;            // codebook entries per pass (multiple of 64, <= kCbsMaxSlice)
  int passes;           // slices covering the 65,536 entries
  float r0;             // stage scale (1 without)
  const uint8_t *idx8;  // a residual stage of 8-bit indices [n][G], or null: none
  const uint16_t *cb8;  // its fp16 codebook [256][8]
  const uint16_t *idx2; // or a second stage of 16-bit indices [n][G], or null: none
  const uint16_t *cb2;  // its fp16 codebook [65536][8]
  float r1;             // the second stage's scale (nonzero with idx2)
  const int8_t *signs;  // the input transform's signs, or null: none
  int mb;               // its largest block
};

// offset = (16-bit half h of p) * 16 + c (mod 2^32): v_mad_u32_u16, whose
// op_sel picks the half, so no instruction extracts it.
template <int H>
__device__ __forceinline__ uint32_t mad16(uint32_t p, uint32_t c) {
  uint32_t r;
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (H) asm("v_mad_u32_u16 %0, %1, 16, %2 op_sel:[1,0,0,0]" : "=v"(r) : "v"(p), "s"(c));
  else asm("v_mad_u32_u16 %0, %1, 16, %2" : "=v"(r) : "v"(p), "s"(c));
#else
  r = (H ? p >> 16 : p & 0xffffu) * 16u + c;
#endif
  return r;
}

// f(integral_constant<int, I>) for I = B .. E - 1, so each call sees I as a
// compile-time constant (the wait counts below need immediates).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ float dot8(const uint4 c, const uint32_t (&x)[4], float acc) {
  acc = __builtin_amdgcn_fdot2(as_h2(c.x), as_h2(x[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(c.y), as_h2(x[1]), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(c.z), as_h2(x[2]), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(c.w), as_h2(x[3]), acc, false);
  return acc;
}

// MODE 0: one 16-bit stage; 1: plus an 8-bit residual stage (RES); 2: plus
// a second 16-bit stage (ST2), streamed through the slices after the first.
template <int U, int ROWS, int MODE>
__global__ __launch_bounds__(kCbsWaves * 64) void k_gemv_cbs(CbsArgs a) {
  constexpr bool RES = MODE == 1, ST2 = MODE == 2;
  __shared__ uint4 s_cb[kCbsMaxSlice + 1];
  __shared__ uint4 s_res[RES ? 256 : 1];  // the residual stage's codebook (4 KiB beside the slice)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kpart = wave % a.kp;
  const int rset = wave / a.kp;
  const int nrs = kCbsWaves / a.kp;  // row sets
  const int blk_lo = blockIdx.x * a.per_wg;
  const int blk_hi = min(a.n, blk_lo + a.per_wg);
  // rows of this wave: blk_lo + rset + nrs i, i < nr (wave-uniform)
  const int nr = blk_lo + rset < blk_hi ? (blk_hi - 1 - blk_lo - rset) / nrs + 1 : 0;
  // row chunks: the same count for every wave, so every wave meets every barrier
  const int rows_max = (a.per_wg + nrs - 1) / nrs;
  const int chunks = (rows_max + ROWS - 1) / ROWS;
  const uint32_t zero_off = 16u * (uint32_t)a.slice;  // the all-zero entry after the slice
  if (tid == 0) s_cb[a.slice] = make_uint4(0u, 0u, 0u, 0u);
  // the residual codebook lands with the first barrier (LDS-direct copies
  // among the outstanding loads make it wait for all of them)
  if constexpr (RES)
    if (wave < 4) lds_direct_16(reinterpret_cast<const uint4 *>(a.cb8) + wave * 64 + lane, s_res + wave * 64);

  const buf_t bidx = make_buf(a.idx, 2u * (uint32_t)a.n * (uint32_t)a.G);
  const buf_t bidx2 = make_buf(ST2 ? a.idx2 : a.idx, 2u * (uint32_t)a.n * (uint32_t)a.G);
  const uint32_t pair0 = (uint32_t)(kpart * 64 * U + lane);  // the lane's first pair of a row
  const uint4 *cb = reinterpret_cast<const uint4 *>(a.cb);

  // Slice p into LDS: 64 entries per wave and LDS-direct load (lane l's 16
  // bytes at the wave's LDS base + 16 l).  The last slice may end early:
  // lanes past entry 65535 reload it into slots no index reaches.
  auto stage = [&](int p, const uint4 *cbp) {
    const int e0 = p * a.slice;
    for (int c = wave; c * 64 < a.slice; c += kCbsWaves) {  // wave-uniform
      const int e = min(e0 + c * 64 + lane, 65535);
      lds_direct_16(cbp + e, s_cb + c * 64);
    }
  };

  // x of the lane's pairs, fp16 after a power-of-two rescale that puts the
  // largest |x| of the lane's 16 U values in [2^14, 2^15); f undoes it.
  uint32_t X[U][2][4];
  float f;
  {
    float xv[U][16];
    if (a.signs) {
      // The input transform (GLQ page, "How it works": random sign flips,
      // then a fast Walsh-Hadamard transform, block-diagonal over the greedy
      // power-of-two blocks of at most mb, "Bit widths"), on this
      // workgroup's fp32 copy of x in the LDS that slice 0 later takes: the
      // signs multiply x as it is staged (with blocks of at least 32, 16
      // consecutive elements per thread and their first four butterfly
      // stages in registers), then passes of butterfly stages, each block
      // scaled by 1/sqrt(its length) in its last pass.
      constexpr int NT = kCbsWaves * 64;
      float *s_x = reinterpret_cast<float *>(s_cb);
      const bool rht16 = a.mb >= 32;  // uniform
      if (rht16) {
        for (int g = tid; g < a.k / 16; g += NT) {
          float v[16];
          rht_load16(a.x, a.xt == VQ_F32, a.signs, 16 * g, v);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(&s_x[16 * g + 4 * q]) =
                make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      } else {
        for (int i = tid; i < a.k; i += NT) {
          const float v = a.xt == VQ_F32 ? reinterpret_cast<const float *>(a.x)[i]
                                         : bf2f(reinterpret_cast<const uint16_t *>(a.x)[i]);
          s_x[i] = v * (float)a.signs[i];
        }
      }
      fwht_lds<NT>(s_x, a.k, a.mb, tid, rht16 ? 4 : 0);
      __syncthreads();  // the last pass is complete
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t = *reinterpret_cast<const float4 *>(&s_x[16 * (pair0 + 64u * j) + 4 * q]);
          xv[j][4 * q] = t.x, xv[j][4 * q + 1] = t.y, xv[j][4 * q + 2] = t.z, xv[j][4 * q + 3] = t.w;
        }
      __syncthreads();  // every lane holds its values before slice 0 overwrites them
    } else if (a.xt == VQ_F32) {
      // every load of the lane's x issued before the first use (one branch
      // on the dtype around all of them)
      float4 t[U][4];
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          t[j][q] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + 16 * (pair0 + 64u * j))[q];
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[j][4 * q] = t[j][q].x, xv[j][4 * q + 1] = t[j][q].y;
          xv[j][4 * q + 2] = t[j][q].z, xv[j][4 * q + 3] = t[j][q].w;
        }
    } else {
      uint4 t[U][2];
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          t[j][q] = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.x) + 16 * (pair0 + 64u * j))[q];
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t w4[4] = {t[j][q].x, t[j][q].y, t[j][q].z, t[j][q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[j][8 * q + 2 * e] = bf2f(w4[e] & 0xffffu);
            xv[j][8 * q + 2 * e + 1] = bf2f(w4[e] >> 16);
          }
        }
    }
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(xv[j][e]));
    const int xexp = (mx > 0.f && mx <= 3.0e38f) ? 14 - ilogbf(mx) : 0;
    f = ldexpf(1.f, -xexp);
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const half2_t v = half2_t{(_Float16)ldexpf(xv[j][8 * h + 2 * e], xexp),
                                    (_Float16)ldexpf(xv[j][8 * h + 2 * e + 1], xexp)};
          X[j][h][e] = __builtin_bit_cast(uint32_t, v);
        }
  }

  uint32_t I[ROWS][U];
  float acc[ROWS];

  // A batch is half a row: the low (h = 0) or the high (h = 1) index of
  // each of the row's U pairs.  issue: the batch's U indices against slice p
  // (offset constant c = -16 p S) as 16-byte LDS reads; consume: their dot
  // products in a fixed order.  The registers of I are made opaque first:
  // nothing computed from them is hoisted out of the pass loop (that would
  // keep 2U offsets per row live across it).
  auto issue = [&](int i, int h, uint32_t c, uint4 (&v)[U]) {
#pragma unroll
    for (int j = 0; j < U; ++j) asm volatile("" : "+v"(I[i][j]));
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t o = min(h ? mad16<1>(I[i][j], c) : mad16<0>(I[i][j], c), zero_off);
      v[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(s_cb) + o);
    }
  };
  auto consume = [&](int i, int h, const uint4 (&v)[U]) {
#pragma unroll
    for (int j = 0; j < U; ++j) acc[i] = dot8(v[j], X[j][h], acc[i]);
  };
  // One pass over the 2 ROWS batches of rows 0 .. ROWS-1: batch b+1's reads
  // are issued before batch b's dot products (two batches' vectors live,
  // 8U registers).  In pass 0 (first) a row's first batch waits for that
  // row's index loads only.
  auto pass = [&](uint32_t c, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    uint4 va[U], vb[U];
    static_for<0, 2 * ROWS>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      constexpr int i = b / 2, h = b % 2;
      constexpr int i1 = (b + 1) / 2, h1 = (b + 1) % 2;
      constexpr int later1 = (ROWS - 1 - i1) * U;  // index loads issued after row i1
      uint4(&cur)[U] = (b & 1) ? vb : va;
      uint4(&nxt)[U] = (b & 1) ? va : vb;
      sched_fence();
      if constexpr (b == 0) {
        if constexpr (kFirst) wait_vmem<((ROWS - 1) * U < 63 ? (ROWS - 1) * U : 63)>();
        issue(0, 0, c, cur);
      }
      if constexpr (b + 1 < 2 * ROWS) {
        if constexpr (kFirst && h1 == 0) wait_vmem<(later1 < 63 ? later1 : 63)>();
        issue(i1, h1, c, nxt);
      }
      sched_fence();
      consume(i, h, cur);
    });
    sched_fence();
  };

  for (int ch = 0; ch < chunks; ++ch) {
    const int i0 = ch * ROWS;                    // the chunk's first row (of this wave's)
    const int nrc = min(ROWS, max(nr - i0, 0));  // this wave's rows in the chunk (uniform)
    if (ch > 0) __syncthreads();  // the previous chunk's last slice and partials are done with
    // Slice 0 lands before the index loads are issued: the barrier's release
    // fence waits for every outstanding load once the LDS-direct copies are
    // among them, so only the slice is outstanding here.
    stage(0, cb);
    __syncthreads();
    // index loads of the chunk's rows (past the wave's last row: that row
    // again, or any valid row for a wave without rows; never used)
    auto load_idx = [&](const buf_t bi) {
#pragma unroll
      for (int i = 0; i < ROWS; ++i) {
        const int ri = min(blk_lo + rset + nrs * min(i0 + i, max(nr - 1, 0)), a.n - 1);
        const uint32_t rb = 2u * (uint32_t)ri * (uint32_t)a.G;
#pragma unroll
        for (int j = 0; j < U; ++j) I[i][j] = buf_u32(bi, 4u * (pair0 + 64u * j), rb);
      }
      sched_fence();
    };
    load_idx(bidx);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) acc[i] = 0.f;
    // Pass 0 takes each row as its indices arrive (the loads after row i
    // may still be in flight), so it overlaps the index stream from HBM.
    // Every pass runs all ROWS rows without a branch (rows past the wave's
    // last are duplicates whose sums are dropped): guarded rows let the
    // compiler defer every row's dot products to a join block and keep all
    // the gathered vectors live.
    // One copy of the pass code serves every pass: its waits for the index
    // loads are no-ops once the loads have landed, and a single copy keeps
    // the code small (about 28 KiB) and the 7-pair instance free of spills.
    // With a second 16-bit stage (ST2) its slices follow the first stage's;
    // at the switch its indices are loaded into the same registers, and the
    // row sums so far are multiplied by r0 / r1, so that the stages share one
    // accumulator and the final r1 gives r0 (stage 0) + r1 (stage 1).
    const int npass = ST2 ? 2 * a.passes : a.passes;
    for (int q = 0; q < npass; ++q) {
      int p = q;
      if constexpr (ST2) p = q < a.passes ? q : q - a.passes;
      if (q > 0) {
        __syncthreads();  // every wave is done with the previous slice
        if constexpr (ST2) stage(p, q < a.passes ? cb : reinterpret_cast<const uint4 *>(a.cb2));
        else stage(p, cb);
        wait_vmem<0>();
        __syncthreads();
        if constexpr (ST2) {
          if (q == a.passes) {  // uniform
            load_idx(bidx2);
            const float fold = a.r0 / a.r1;
#pragma unroll
            for (int i = 0; i < ROWS; ++i) acc[i] *= fold;
          }
        }
      }
      pass(0u - 16u * (uint32_t)(p * a.slice), std::true_type{});
    }
    // The residual stage (GLQ page, "Advanced > Bit widths": a 16-bit primary
    // plus an 8-bit residual; each stage's sum times its stage scale): one
    // more pass over the codebook in LDS, its index bytes (the pair's two
    // groups in one 16-bit load) loaded now into the registers the 16-bit
    // indices held, each row taken as its loads land.
    float acc1[RES ? ROWS : 1];
    if constexpr (RES) {
      const buf_t bres = make_buf(a.idx8, (uint32_t)a.n * (uint32_t)a.G);
      uint32_t R[ROWS][U];
#pragma unroll
      for (int i = 0; i < ROWS; ++i) {
        const int ri = min(blk_lo + rset + nrs * min(i0 + i, max(nr - 1, 0)), a.n - 1);
        const uint32_t rb = (uint32_t)ri * (uint32_t)a.G;
#pragma unroll
        for (int j = 0; j < U; ++j) R[i][j] = buf_u16(bres, 2u * (pair0 + 64u * j), rb);
        acc1[i] = 0.f;
      }
      sched_fence();
      static_for<0, ROWS>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int later = (ROWS - 1 - i) * U;  // loads issued after row i
        wait_vmem<(later < 63 ? later : 63)>();
        uint4 v[2][U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          v[0][j] = s_res[R[i][j] & 0xffu];
          v[1][j] = s_res[(R[i][j] >> 8) & 0xffu];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
          acc1[i] = dot8(v[0][j], X[j][0], acc1[i]);
          acc1[i] = dot8(v[1][j], X[j][1], acc1[i]);
        }
        // the sum is made here: left free, the compiler sinks the dot
        // products into the guarded reduction and keeps every gathered
        // vector live until then
        asm volatile("" : "+v"(acc1[i]));
        sched_fence();
      });
    }
    // Per row: the lane's sum times its rescale factor, reduced across the
    // wave in a fixed order; the K parts of a row are then added in order
    // 0, 1, ... through LDS, times the row scale.
    __syncthreads();  // every wave is done with the last slice
    float *s_part = reinterpret_cast<float *>(s_cb);  // [row set][K part][ROWS]
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      if (i < nrc) {
        float ai = acc[i];
        if constexpr (RES) ai = a.r0 * acc[i] + a.r1 * acc1[i];  // each stage's sum times its scale
        const float t = wave_sum(ai * f);
        if (lane == 0) s_part[(rset * a.kp + kpart) * ROWS + i] = t;
      }
    }
    __syncthreads();
    // thread t: row t of the workgroup's chunk rows (row set t % nrs, index t / nrs)
    for (int t = tid; t < nrs * ROWS; t += kCbsWaves * 64) {
      const int rs = t % nrs, i = t / nrs;
      const int row_i = i0 + i;  // index within row set rs
      const int nr_rs = blk_lo + rs < blk_hi ? (blk_hi - 1 - blk_lo - rs) / nrs + 1 : 0;
      if (row_i < nr_rs) {
        float s = 0.f;
        for (int q = 0; q < a.kp; ++q) s += s_part[(rs * a.kp + q) * ROWS + i];
        const int r = blk_lo + rs + nrs * row_i;
        a.y[r] = s * (h2f(a.sc[r]) * (RES ? 1.f : ST2 ? a.r1 : a.r0));
      }
    }
  }
}

// Rows per wave (index registers ROWS x U <= 112) for each pairs-per-lane U.
template <int U> constexpr int cbs_rows() { return U <= 2 ? 32 : U == 8 ? 12 : 112 / U; }


template <int U>
void launch_u(const CbsArgs &a0, int cus, hipStream_t s) {
  CbsArgs a = a0;
  const int nrs = kCbsWaves / a.kp;
  int grid = (a.n + nrs - 1) / nrs;  // at least one row per row set where possible
  if (grid > cus) grid = cus;
  a.per_wg = (a.n + grid - 1) / grid;
  if (a.idx8) hipLaunchKernelGGL((k_gemv_cbs<U, cbs_rows<U>(), 1>), dim3(grid), dim3(kCbsWaves * 64), 0, s, a);
  else if (a.idx2) hipLaunchKernelGGL((k_gemv_cbs<U, cbs_rows<U>(), 2>), dim3(grid), dim3(kCbsWaves * 64), 0, s, a);
  else hipLaunchKernelGGL((k_gemv_cbs<U, cbs_rows<U>(), 0>), dim3(grid), dim3(kCbsWaves * 64), 0, s, a);
}

// Largest K whose fp32 copy fits the LDS for the in-kernel input transform.
constexpr int kCbsMaxRhtK = 4 * kCbsMaxSlice;

// Pairs per lane and K part for K = 1024 ppr: U divides ppr into 1, 2, 4 or
// 8 K parts (8 waves), 4 preferred (x and indices both fit the registers
// best), then 7, 8, 2, 1; 0 when none does.
int cbs_pairs(int k) {
  if (k % 1024) return 0;
  const int ppr = k / 1024;
  for (int u : {4, 7, 8, 2, 1}) {
    if (ppr % u) continue;
    const int kp = ppr / u;
    if (kp == 1 || kp == 2 || kp == 4 || kp == 8) return u;
  }
  return 0;
}

}  // namespace

bool gemv_cbs_takes(const WView &w) {
  const bool two = w.S == 2 && (w.sb[1] == 8 || w.sb[1] == 16);  // an 8- or 16-bit second stage
  if ((w.S != 1 && !two) || w.sb[0] != 16 || w.nblk != 1) return false;
  if ((int64_t)w.n * w.k < ((int64_t)1 << 25)) return false;  // small weights: L2 gathers
  return cbs_pairs(w.k) != 0;
}

bool gemv_cbs_rht_takes(const WView &w) { return gemv_cbs_takes(w) && w.k <= kCbsMaxRhtK; }

bool launch_gemv_cbs(const WView &w, const void *x, int xt, float *y, int cus, hipStream_t s, const int8_t *signs,
                     int max_block) {
  if (!(signs ? gemv_cbs_rht_takes(w) : gemv_cbs_takes(w))) return false;
  const int u = cbs_pairs(w.k);
  CbsArgs a{};
  a.idx = w.i16[0];
  a.cb = w.cb[0];
  a.sc = w.sc;
  a.x = x;
  a.y = y;
  a.xt = xt;
  a.n = w.n;
  a.k = w.k;
  a.G = w.G;
  a.kp = w.k / (1024 * u);
  a.slice = kCbsMaxSlice;
  a.passes = kCbsPasses;
  a.r0 = w.rs[0];
  if (w.S == 2 && w.sb[1] == 8) {  // an 8-bit residual stage (gemv_cbs_takes)
    a.idx8 = w.lo[1];
    a.cb8 = w.cb[1];
    a.r1 = w.rs[1];
  } else if (w.S == 2 && w.rs[1] != 0.f) {  // a second 16-bit stage (one scaled by 0 adds nothing)
    a.idx2 = w.i16[1];
    a.cb2 = w.cb[1];
    a.r1 = w.rs[1];
  }
  a.signs = signs;
  a.mb = max_block;
  switch (u) {
    case 1: launch_u<1>(a, cus, s); break;
    case 2: launch_u<2>(a, cus, s); break;
    case 4: launch_u<4>(a, cus, s); break;
    case 7: launch_u<7>(a, cus, s); break;
    default: launch_u<8>(a, cus, s); break;
  }
  return true;
}

}  // namespace vqmm
