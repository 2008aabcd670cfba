// Decode-path product for one stage of 16-bit indices into a 65,536-entry
// codebook (1 MiB, GLQ page "How it works" / "Bit widths"), which cannot sit
// in LDS: every codebook vector is a 16-byte gather that hits in L2.
//
// k_gemv_l2 -- the gathers are the whole cost, and a gather waits on its
// row's index load from HBM, so the kernel is built to keep many of both in
// flight:
//   * persistent grid, one workgroup of 8 waves per CU owning a contiguous
//     block of rows, each wave every 8th row of it;
//   * lane l owns the 4-group units l + 64 j of every row (8 bytes of
//     indices each, one buffer load; the unit's scale likewise);
//   * the next row's indices and scales load while a row is computed (a
//     two-row ring), so a row's gathers never wait for HBM;
//   * a row's gathers go out 16 per lane (four units) before their dot
//     products with x, which is staged once per workgroup in LDS as fp32;
//   * per unit the 32 products are summed, scaled and accumulated in a fixed
//     order; one fixed-order wave reduction per row.  No atomics.
// Taken for one stage of 16-bit indices, or a 16-bit primary plus one
// residual stage of 8 bits (its 4 KiB codebook in LDS) or 16 bits (L2
// gathers too), optionally with stage scales (GLQ page, "Bit widths": the
// 3 and 4 bpw ladders; "Inference kernels": the inverse residual scale);
// K % 2048 == 0 (K / 2048 units per lane) up to K = 32768 (x in LDS), scale
// blocks of whole 32-column units.
//
// With signs given, the kernel first applies the randomized Hadamard
// transform of the input to its LDS copy of x (GLQ page, "How it works":
// random sign flips, then a fast Walsh-Hadamard transform; "Bit widths":
// block-diagonal over the greedy power-of-two blocks of at most max_block),
// the same transform rht_apply computes: the signs multiply x as it is
// staged, then passes of up to four butterfly stages each run in registers
// over groups of 16 elements (one barrier per pass, every block of the row
// in the same pass), and each block's last pass scales it by 1/sqrt(len).
// Every workgroup transforms its own copy, so no second launch and no
// buffer for the transformed x are needed.
#include "gemv_kernels.h"

namespace vqmm {

namespace {

constexpr int kL2Waves = 8;
constexpr int kL2MaxK = 32768;  // fp32 x in LDS: 128 KiB
// units whose gathers are in flight together (16 per lane either way)
template <int B1> constexpr int l2_batch() { return B1 == 16 ? 2 : 4; }
// most units per lane that fit the register file without spills
template <int B1> constexpr int l2_max_upl() { return B1 == 0 ? 16 : B1 == 8 ? 14 : 13; }

// B1: width of the residual stage (0: none, 8 or 16); RS: stage scales.
template <int UPL, int B1, bool RS>
__global__ __launch_bounds__(kL2Waves * 64) void k_gemv_l2(GemvArgs a, int xt, RhtIn rht) {
  constexpr int NT = kL2Waves * 64;
  __shared__ float s_x[kL2MaxK];
  __shared__ uint4 s_cb1[B1 == 8 ? 256 : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int K = a.k;

  // x -> LDS as fp32 (times the signs of the input transform), four values
  // per thread and step.  With the transform and blocks of at least 32
  // elements (K % 2048 == 0, so every block then is), a thread stages 16
  // consecutive elements and runs the transform's first four butterfly
  // stages on them in registers.
  const bool has_rht = rht.signs != nullptr;  // uniform
  const bool rht16 = has_rht && rht.mb >= 32;
  if (rht16) {
    for (int g = tid; g < K / 16; g += NT) {
      float v[16];
      rht_load16(a.x, xt == VQ_F32, rht.signs, 16 * g, v);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(&s_x[16 * g + 4 * q]) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
  }
  for (int i = 4 * tid; i < (rht16 ? 0 : K); i += 4 * NT) {
    float4 v;
    if (xt == VQ_F32) {
      v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + i);
    } else {
      const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.x) + i);
      v = make_float4(bf2f(u.x & 0xffffu), bf2f(u.x >> 16), bf2f(u.y & 0xffffu), bf2f(u.y >> 16));
    }
    if (has_rht) {
      const uint32_t sg = *reinterpret_cast<const uint32_t *>(rht.signs + i);
      v.x *= (float)(int8_t)(sg & 0xffu);
      v.y *= (float)(int8_t)((sg >> 8) & 0xffu);
      v.z *= (float)(int8_t)((sg >> 16) & 0xffu);
      v.w *= (float)(int8_t)(sg >> 24);
    }
    *reinterpret_cast<float4 *>(&s_x[i]) = v;
  }
  if (B1 == 8 && tid < 256) s_cb1[tid] = reinterpret_cast<const uint4 *>(a.cb[1])[tid];
  if (has_rht) fwht_lds<NT>(s_x, K, rht.mb, tid, rht16 ? 4 : 0);
  __syncthreads();  // the last barrier: waves without rows may leave after it

  const int per_wg = (a.n + gridDim.x - 1) / gridDim.x;
  const int blk_lo = blockIdx.x * per_wg;
  const int blk_hi = min(a.n, blk_lo + per_wg);
  const int row0 = blk_lo + wave;
  const int nrows = row0 < blk_hi ? (blk_hi - 1 - row0) / kL2Waves + 1 : 0;  // wave-uniform
  if (nrows == 0) return;

  const uint32_t G = (uint32_t)a.G;
  const buf_t bi = make_buf(a.i16[0], 2u * (uint32_t)a.n * G);
  const buf_t bsc = make_buf(a.sc, 2u * (uint32_t)a.n * (uint32_t)a.nblk);
  const buf_t bcb = make_buf(a.cb[0], 65536u * 16u);
  const buf_t bi1 = make_buf(B1 == 16 ? (const void *)a.i16[1] : (const void *)a.lo[1], (B1 == 16 ? 2u : 1u) * (uint32_t)a.n * G);
  const buf_t bcb1 = make_buf(a.cb[1], 65536u * 16u);
  const float r0 = RS ? a.rs[0] : 1.f, r1 = RS ? a.rs[1] : 1.f;
  // Unit lane + 64 j (4 groups = 32 columns) sits at byte 8 lane + 512 j of a
  // row of 16-bit indices; its scale at 2 ((32 lane + 2048 j) / bs), which
  // splits into a lane part and a wave-uniform part because bs divides 2048
  // or is at least K (then every unit has scale 0 of its row).
  constexpr int kBatch = l2_batch<B1>();
  const uint32_t bs = (uint32_t)a.bs;
  const uint32_t vsc = 2u * ((32u * (uint32_t)lane) / bs);
  const uint32_t sstep = 2u * (2048u / bs);

  struct RowI {
    uint2 I[UPL];
    uint32_t S[UPL];
    uint2 I1[B1 ? UPL : 1];  // residual indices (8-bit: four bytes in .x)
  };
  auto load_row = [&](int r, RowI &R) {
    // past the wave's last row: that row again (an L2 hit, never stored)
    const uint32_t rr = (uint32_t)(row0 + min(r, nrows - 1) * kL2Waves);
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      R.I[j] = buf_u64(bi, 8u * lane, 2u * rr * G + 512u * j);
      R.S[j] = buf_u16(bsc, vsc, 2u * rr * (uint32_t)a.nblk + sstep * j);
      if constexpr (B1 == 16) R.I1[j] = buf_u64(bi1, 8u * lane, 2u * rr * G + 512u * j);
      if constexpr (B1 == 8) R.I1[j] = make_uint2(buf_u32(bi1, 4u * lane, rr * G + 256u * j), 0u);
    }
  };
  auto compute_row = [&](int r, const RowI &R) {
    float acc = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < UPL; j0 += kBatch) {
      uint4 cv[kBatch][4];
      uint4 cv1[B1 == 16 ? kBatch : 1][4];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        if (j0 + jj < UPL) {
          const uint2 w = R.I[j0 + jj];
          cv[jj][0] = buf_u128(bcb, (w.x & 0xffffu) << 4, 0);
          cv[jj][1] = buf_u128(bcb, (w.x >> 16) << 4, 0);
          cv[jj][2] = buf_u128(bcb, (w.y & 0xffffu) << 4, 0);
          cv[jj][3] = buf_u128(bcb, (w.y >> 16) << 4, 0);
          if constexpr (B1 == 16) {
            const uint2 w1 = R.I1[j0 + jj];
            cv1[jj][0] = buf_u128(bcb1, (w1.x & 0xffffu) << 4, 0);
            cv1[jj][1] = buf_u128(bcb1, (w1.x >> 16) << 4, 0);
            cv1[jj][2] = buf_u128(bcb1, (w1.y & 0xffffu) << 4, 0);
            cv1[jj][3] = buf_u128(bcb1, (w1.y >> 16) << 4, 0);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        if (j0 + jj < UPL) {
          const int col0 = 32 * (lane + 64 * (j0 + jj));
          // products of one stage's vector with the 8 x of group q
          auto dot8 = [&](const uint4 c, const float4 x0, const float4 x1, float d) {
            d = fmaf(h2f(c.x & 0xffffu), x0.x, d);
            d = fmaf(h2f(c.x >> 16), x0.y, d);
            d = fmaf(h2f(c.y & 0xffffu), x0.z, d);
            d = fmaf(h2f(c.y >> 16), x0.w, d);
            d = fmaf(h2f(c.z & 0xffffu), x1.x, d);
            d = fmaf(h2f(c.z >> 16), x1.y, d);
            d = fmaf(h2f(c.w & 0xffffu), x1.z, d);
            d = fmaf(h2f(c.w >> 16), x1.w, d);
            return d;
          };
          float d = 0.f, d1 = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 x0 = *reinterpret_cast<const float4 *>(&s_x[col0 + 8 * q]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&s_x[col0 + 8 * q + 4]);
            d = dot8(cv[jj][q], x0, x1, d);
            if constexpr (B1 == 16) d1 = dot8(cv1[jj][q], x0, x1, d1);
            if constexpr (B1 == 8) d1 = dot8(s_cb1[(R.I1[j0 + jj].x >> (8 * q)) & 0xffu], x0, x1, d1);
          }
          // residual: its own sum, then the stage scales (1 without them)
          if (B1 || RS) d = B1 ? fmaf(r1, d1, r0 * d) : r0 * d;
          acc = fmaf(h2f(R.S[j0 + jj]), d, acc);
        }
      }
    }
    const float tot = wave_sum(acc);
    if (lane == 0) a.y[row0 + r * kL2Waves] = tot;
  };

  RowI R0, R1;
  load_row(0, R0);
  int r = 0;
  for (; r + 2 <= nrows; r += 2) {
    load_row(r + 1, R1);
    sched_fence();
    compute_row(r, R0);
    load_row(r + 2, R0);
    sched_fence();
    compute_row(r + 1, R1);
  }
  if (r < nrows) compute_row(r, R0);
}

template <int UPL, int B1, bool RS>
bool launch_u(const GemvArgs &a, int xt, RhtIn rht, int cus, hipStream_t s) {
  if constexpr (UPL > l2_max_upl<B1>()) {
    return false;
  } else {
    int g = (a.n + kL2Waves - 1) / kL2Waves;
    if (g > cus) g = cus;
    hipLaunchKernelGGL((k_gemv_l2<UPL, B1, RS>), dim3(g), dim3(kL2Waves * 64), 0, s, a, xt, rht);
    return true;
  }
}

template <int B1, bool RS>
bool launch_f(const GemvArgs &a, int xt, RhtIn rht, int cus, hipStream_t s) {
  switch (a.k / 2048) {
    case 1: return launch_u<1, B1, RS>(a, xt, rht, cus, s);
    case 2: return launch_u<2, B1, RS>(a, xt, rht, cus, s);
    case 3: return launch_u<3, B1, RS>(a, xt, rht, cus, s);
    case 4: return launch_u<4, B1, RS>(a, xt, rht, cus, s);
    case 5: return launch_u<5, B1, RS>(a, xt, rht, cus, s);
    case 6: return launch_u<6, B1, RS>(a, xt, rht, cus, s);
    case 7: return launch_u<7, B1, RS>(a, xt, rht, cus, s);
    case 8: return launch_u<8, B1, RS>(a, xt, rht, cus, s);
    case 9: return launch_u<9, B1, RS>(a, xt, rht, cus, s);
    case 10: return launch_u<10, B1, RS>(a, xt, rht, cus, s);
    case 11: return launch_u<11, B1, RS>(a, xt, rht, cus, s);
    case 12: return launch_u<12, B1, RS>(a, xt, rht, cus, s);
    case 13: return launch_u<13, B1, RS>(a, xt, rht, cus, s);
    case 14: return launch_u<14, B1, RS>(a, xt, rht, cus, s);
    case 15: return launch_u<15, B1, RS>(a, xt, rht, cus, s);
    case 16: return launch_u<16, B1, RS>(a, xt, rht, cus, s);
    default: return false;
  }
}

}  // namespace

bool gemv_l2_takes(const WView &w) {
  if (w.S < 1 || w.S > 2 || w.sb[0] != 16) return false;
  if (w.k % 2048 != 0 || w.k > kL2MaxK) return false;
  if (w.bs % 32 != 0 || (2048 % w.bs != 0 && w.bs < w.k)) return false;
  const int b1 = w.S == 2 ? w.sb[1] : 0;
  if (b1 != 0 && b1 != 8 && b1 != 16) return false;
  const int upl = w.k / 2048;
  return upl <= (b1 == 0 ? l2_max_upl<0>() : b1 == 8 ? l2_max_upl<8>() : l2_max_upl<16>());
}

bool launch_gemv_l2(const WView &w, const GemvArgs &a, int xt, int cus, hipStream_t s, const int8_t *signs,
                    int max_block) {
  if (!gemv_l2_takes(w)) return false;
  const RhtIn rht{signs, max_block};
  const int b1 = w.S == 2 ? w.sb[1] : 0;
  if (!w.scaled) {
    if (b1 == 0) return launch_f<0, false>(a, xt, rht, cus, s);
    return b1 == 8 ? launch_f<8, false>(a, xt, rht, cus, s) : launch_f<16, false>(a, xt, rht, cus, s);
  }
  if (b1 == 0) return launch_f<0, true>(a, xt, rht, cus, s);
  return b1 == 8 ? launch_f<8, true>(a, xt, rht, cus, s) : launch_f<16, true>(a, xt, rht, cus, s);
}

}  // namespace vqmm
