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
// Taken for one stage of 16-bit indices, K % 2048 == 0 (K / 2048 units per
// lane) up to K = 32768 (x in LDS), scale blocks of whole 32-column units.
#include "gemv_kernels.h"

namespace vqmm {

namespace {

constexpr int kL2Waves = 8;
constexpr int kL2MaxK = 32768;  // fp32 x in LDS: 128 KiB
constexpr int kL2Batch = 4;     // units whose gathers are in flight together

template <int UPL>
__global__ __launch_bounds__(kL2Waves * 64) void k_gemv_l2(GemvArgs a, int xt) {
  constexpr int NT = kL2Waves * 64;
  __shared__ float s_x[kL2MaxK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int K = a.k;

  // x -> LDS as fp32, four values per thread and step
  for (int i = 4 * tid; i < K; i += 4 * NT) {
    float4 v;
    if (xt == VQ_F32) {
      v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + i);
    } else {
      const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.x) + i);
      v = make_float4(bf2f(u.x & 0xffffu), bf2f(u.x >> 16), bf2f(u.y & 0xffffu), bf2f(u.y >> 16));
    }
    *reinterpret_cast<float4 *>(&s_x[i]) = v;
  }
  __syncthreads();  // the only barrier: waves without rows may leave after it

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
  uint32_t vu[UPL], vs[UPL];
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const uint32_t u = (uint32_t)(lane + 64 * j);  // unit of 4 groups = 32 columns
    vu[j] = 8u * u;
    vs[j] = 2u * ((32u * u) / (uint32_t)a.bs);
  }

  struct RowI {
    uint2 I[UPL];
    uint32_t S[UPL];
  };
  auto load_row = [&](int r, RowI &R) {
    // past the wave's last row: that row again (an L2 hit, never stored)
    const uint32_t rr = (uint32_t)(row0 + min(r, nrows - 1) * kL2Waves);
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      R.I[j] = buf_u64(bi, vu[j], 2u * rr * G);
      R.S[j] = buf_u16(bsc, vs[j], 2u * rr * (uint32_t)a.nblk);
    }
  };
  auto compute_row = [&](int r, const RowI &R) {
    float acc = 0.f;
#pragma unroll
    for (int j0 = 0; j0 < UPL; j0 += kL2Batch) {
      uint4 cv[kL2Batch][4];
#pragma unroll
      for (int jj = 0; jj < kL2Batch; ++jj) {
        if (j0 + jj < UPL) {
          const uint2 w = R.I[j0 + jj];
          cv[jj][0] = buf_u128(bcb, (w.x & 0xffffu) << 4, 0);
          cv[jj][1] = buf_u128(bcb, (w.x >> 16) << 4, 0);
          cv[jj][2] = buf_u128(bcb, (w.y & 0xffffu) << 4, 0);
          cv[jj][3] = buf_u128(bcb, (w.y >> 16) << 4, 0);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kL2Batch; ++jj) {
        if (j0 + jj < UPL) {
          const int col0 = 32 * (lane + 64 * (j0 + jj));
          float d = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 x0 = *reinterpret_cast<const float4 *>(&s_x[col0 + 8 * q]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&s_x[col0 + 8 * q + 4]);
            const uint4 c = cv[jj][q];
            d = fmaf(h2f(c.x & 0xffffu), x0.x, d);
            d = fmaf(h2f(c.x >> 16), x0.y, d);
            d = fmaf(h2f(c.y & 0xffffu), x0.z, d);
            d = fmaf(h2f(c.y >> 16), x0.w, d);
            d = fmaf(h2f(c.z & 0xffffu), x1.x, d);
            d = fmaf(h2f(c.z >> 16), x1.y, d);
            d = fmaf(h2f(c.w & 0xffffu), x1.z, d);
            d = fmaf(h2f(c.w >> 16), x1.w, d);
          }
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

template <int UPL>
void launch_u(const GemvArgs &a, int xt, int cus, hipStream_t s) {
  int g = (a.n + kL2Waves - 1) / kL2Waves;
  if (g > cus) g = cus;
  hipLaunchKernelGGL((k_gemv_l2<UPL>), dim3(g), dim3(kL2Waves * 64), 0, s, a, xt);
}

}  // namespace

bool launch_gemv_l2(const WView &w, const GemvArgs &a, int xt, int cus, hipStream_t s) {
  if (!plain_format(w) || w.bits != 16 || w.S != 1) return false;
  if (w.k % 2048 != 0 || w.k > kL2MaxK || w.bs % 32 != 0) return false;
  switch (w.k / 2048) {
    case 1: launch_u<1>(a, xt, cus, s); return true;
    case 2: launch_u<2>(a, xt, cus, s); return true;
    case 3: launch_u<3>(a, xt, cus, s); return true;
    case 4: launch_u<4>(a, xt, cus, s); return true;
    case 5: launch_u<5>(a, xt, cus, s); return true;
    case 6: launch_u<6>(a, xt, cus, s); return true;
    case 7: launch_u<7>(a, xt, cus, s); return true;
    case 8: launch_u<8>(a, xt, cus, s); return true;
    case 9: launch_u<9>(a, xt, cus, s); return true;
    case 10: launch_u<10>(a, xt, cus, s); return true;
    case 11: launch_u<11>(a, xt, cus, s); return true;
    case 12: launch_u<12>(a, xt, cus, s); return true;
    case 13: launch_u<13>(a, xt, cus, s); return true;
    case 14: launch_u<14>(a, xt, cus, s); return true;
    case 15: launch_u<15>(a, xt, cus, s); return true;
    case 16: launch_u<16>(a, xt, cus, s); return true;
    default: return false;
  }
}

}  // namespace vqmm
