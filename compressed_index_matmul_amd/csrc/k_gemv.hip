// Decode-path product y = x dequant(W)^T for one token (GLQ page, "Inference
// kernels": each output row walks its K/8 codebook groups, gathering 8-wide
// codebook vectors, and accumulates against the indices without forming W;
// split-K-style lane partials reduced inside the wave in a fixed order).
//
// k_gemv_lds  -- codebooks that fit in LDS (8/12-bit, S * 2^b * 16 B <= 128 KiB),
//                K % 32 == 0, scale_block % 32 == 0, K <= 16384.
//   * persistent grid, one workgroup per CU slot; every workgroup stages the
//     codebooks into LDS once and walks rows (one row per wave at a time);
//   * lane l owns the 4-group chunks c = l + 64 j of every row, so its slice of
//     x stays in registers for the whole launch;
//   * per chunk and stage the lane loads one dword of the low-byte plane and
//     one short of the high-nibble plane (coalesced 256 B + 128 B per wave),
//     the next row's loads are issued before the current row is computed;
//   * bf16 x is held as fp16 after a per-lane power-of-two rescale (exact for
//     values within 2^28 of the lane's largest |x|), so a group-stage costs
//     one 16-byte LDS gather and four v_dot2_f32_f16; fp32 x uses v_fma_mix;
//   * the lane partial is scaled per chunk, un-rescaled, and summed across
//     the wave with DPP (fixed order, no atomics).
//
// k_gemv_gen  -- everything else (16-bit indices into a 1 MiB codebook, 3-4
//                12-bit stages, ragged K or scale blocks): codebook rows are
//                gathered from global memory (L2-resident), x is staged in
//                LDS as fp32, one wave per row, lane = 4 consecutive groups
//                when K % 32 == 0, else one group.
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
};

// ---------------------------------------------------------------------------
// fast path
// ---------------------------------------------------------------------------
template <int S, int BITS, int CPL, int WAVES, bool XF16>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_lds(GemvArgs a) {
  __shared__ uint4 s_cb[S << BITS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int stride = gridDim.x * WAVES;
  int row = blockIdx.x * WAVES + wave;

  uint32_t L[CPL][S], H[CPL][S];
  float SC[CPL];

#define VQ_LOAD_ROW(R_, L_, H_, SC_)                                                         \
  {                                                                                          \
    const size_t rb = (size_t)(R_) * a.G;                                                    \
    _Pragma("unroll") for (int j = 0; j < CPL; ++j) {                                        \
      const int c = lane + 64 * j;                                                           \
      if (c < a.C) {                                                                         \
        _Pragma("unroll") for (int t = 0; t < S; ++t) {                                      \
          L_[j][t] = *reinterpret_cast<const uint32_t *>(a.lo[t] + rb + 4 * c);              \
          if (BITS == 12)                                                                    \
            H_[j][t] = *reinterpret_cast<const uint16_t *>(a.hi[t] + (rb >> 1) + 2 * c);     \
          else                                                                               \
            H_[j][t] = 0;                                                                    \
        }                                                                                    \
        SC_[j] = h2f(a.sc[(size_t)(R_) * a.nblk + (32 * c) / a.bs]);                         \
      } else {                                                                               \
        _Pragma("unroll") for (int t = 0; t < S; ++t) { L_[j][t] = 0; H_[j][t] = 0; }        \
        SC_[j] = 0.f;                                                                        \
      }                                                                                      \
    }                                                                                        \
  }

  if (row < a.n) VQ_LOAD_ROW(row, L, H, SC);

  // stage the codebooks
  for (int i = tid; i < (S << BITS); i += WAVES * 64) {
    s_cb[i] = reinterpret_cast<const uint4 *>(a.cb[i >> BITS])[i & ((1 << BITS) - 1)];
  }

  // this lane's slice of x, held for the whole launch
  half2_t xh[XF16 ? CPL : 1][16];
  float xf[XF16 ? 1 : CPL][32];
  int xexp = 0;
  if (XF16) {
    // pass 1: largest |x| of the lane's slice
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < a.C) {
        const uint4 *px = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.x) + 32 * c);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 u = px[v];
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf2f(w4[e] & 0xffffu)), fabsf(bf2f(w4[e] >> 16))));
        }
      }
    }
    // the largest |x| scaled into [2^14, 2^15): fp16 holds every bf16 value
    // within 2^28 of it exactly
    if (mx > 0.f) xexp = 14 - ilogbf(mx);
    // pass 2: rescale and convert (reloads hit the cache)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
#pragma unroll
      for (int q = 0; q < 16; ++q) xh[j][q] = half2_t{(_Float16)0.f, (_Float16)0.f};
      if (c < a.C) {
        const uint4 *px = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.x) + 32 * c);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 u = px[v];
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            xh[j][4 * v + e] = half2_t{(_Float16)ldexpf(bf2f(w4[e] & 0xffffu), xexp),
                                       (_Float16)ldexpf(bf2f(w4[e] >> 16), xexp)};
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
#pragma unroll
      for (int q = 0; q < 32; ++q) xf[j][q] = 0.f;
      if (c < a.C) {
        const float4 *px = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + 32 * c);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4 u = px[v];
          xf[j][4 * v] = u.x;
          xf[j][4 * v + 1] = u.y;
          xf[j][4 * v + 2] = u.z;
          xf[j][4 * v + 3] = u.w;
        }
      }
    }
  }
  __syncthreads();

  while (row < a.n) {
    const int nrow = row + stride;
    uint32_t L2[CPL][S], H2[CPL][S];
    float SC2[CPL];
    if (nrow < a.n) VQ_LOAD_ROW(nrow, L2, H2, SC2);

    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < a.C) {
        float d = 0.f;
#pragma unroll
        for (int t = 0; t < S; ++t) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t idx = (L[j][t] >> (8 * q)) & 0xffu;
            if (BITS == 12) idx |= ((H[j][t] >> (4 * q)) & 0xfu) << 8;
            const uint4 v = s_cb[(t << BITS) + idx];
            if (XF16) {
              d = __builtin_amdgcn_fdot2(as_h2(v.x), xh[j][4 * q + 0], d, false);
              d = __builtin_amdgcn_fdot2(as_h2(v.y), xh[j][4 * q + 1], d, false);
              d = __builtin_amdgcn_fdot2(as_h2(v.z), xh[j][4 * q + 2], d, false);
              d = __builtin_amdgcn_fdot2(as_h2(v.w), xh[j][4 * q + 3], d, false);
            } else {
              const uint32_t hv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                d = fmaf(h2f(hv[e] & 0xffffu), xf[j][8 * q + 2 * e], d);
                d = fmaf(h2f(hv[e] >> 16), xf[j][8 * q + 2 * e + 1], d);
              }
            }
          }
        }
        acc = fmaf(SC[j], d, acc);
      }
    }
    if (XF16) acc = ldexpf(acc, -xexp);
    const float tot = wave_sum(acc);
    if (lane == 0) a.y[row] = tot;

#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      SC[j] = SC2[j];
#pragma unroll
      for (int t = 0; t < S; ++t) {
        L[j][t] = L2[j][t];
        H[j][t] = H2[j][t];
      }
    }
    row = nrow;
  }
#undef VQ_LOAD_ROW
}

// ---------------------------------------------------------------------------
// general path
// ---------------------------------------------------------------------------
constexpr int kGenWaves = 8;
constexpr int kGenMaxXLds = 32768;  // fp32 x elements staged in LDS (128 KiB)

template <int BITS, int GPL, bool X_LDS>
__global__ __launch_bounds__(kGenWaves * 64) void k_gemv_gen(GemvArgs a, int xt) {
  __shared__ float s_x[X_LDS ? kGenMaxXLds : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
        uint32_t idx[GPL];
        if (GPL == 4) {
          if (BITS == 16) {
            const uint2 v = *reinterpret_cast<const uint2 *>(a.i16[t] + rb + g0);
            idx[0] = v.x & 0xffffu;
            idx[1] = v.x >> 16;
            idx[2] = v.y & 0xffffu;
            idx[3] = v.y >> 16;
          } else {
            const uint32_t lw = *reinterpret_cast<const uint32_t *>(a.lo[t] + rb + g0);
            uint32_t hw = 0;
            if (BITS == 12) hw = *reinterpret_cast<const uint16_t *>(a.hi[t] + ((rb + g0) >> 1));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              idx[q] = (lw >> (8 * q)) & 0xffu;
              if (BITS == 12) idx[q] |= ((hw >> (4 * q)) & 0xfu) << 8;
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < GPL; ++q) idx[q] = load_index(BITS, a.lo[t], a.hi[t], a.i16[t], rb + g0 + q);
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
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d[q] = fmaf(h2f(hv[e] & 0xffffu), xv[2 * e], d[q]);
            d[q] = fmaf(h2f(hv[e] >> 16), xv[2 * e + 1], d[q]);
          }
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
// dispatch
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
  return a;
}

// x lives in registers: up to 8 chunks per lane as fp16 (K <= 16384), up to
// 4 as fp32 (K <= 8192).
bool gemv_fast_eligible(const WView &w, int xt) {
  if (w.bits == 16) return false;
  if ((size_t)(w.S << w.bits) * 16 > 131072) return false;
  if (w.k % 32 || w.bs % 32) return false;
  const int cpl = (w.G / 4 + 63) / 64;
  return cpl <= (xt == VQ_BF16 ? 8 : 4);
}

template <int S, int BITS, int CPL, bool XF16>
static void launch_fast_c(const GemvArgs &a, int cus, hipStream_t s) {
  constexpr int W = CPL <= 2 ? 16 : 8;
  constexpr size_t lds = (size_t)(S << BITS) * 16;
  const int per_cu = lds > 81920 ? 1 : 2;
  int nwg = (a.n + W - 1) / W;
  if (nwg > cus * per_cu) nwg = cus * per_cu;
  hipLaunchKernelGGL((k_gemv_lds<S, BITS, CPL, W, XF16>), dim3(nwg), dim3(W * 64), 0, s, a);
}

template <int S, int BITS, bool XF16>
static void launch_fast_s(const GemvArgs &a, int cus, hipStream_t s) {
  switch ((a.C + 63) / 64) {
    case 1: launch_fast_c<S, BITS, 1, XF16>(a, cus, s); break;
    case 2: launch_fast_c<S, BITS, 2, XF16>(a, cus, s); break;
    case 3: launch_fast_c<S, BITS, 3, XF16>(a, cus, s); break;
    case 4: launch_fast_c<S, BITS, 4, XF16>(a, cus, s); break;
    case 5: if constexpr (XF16) launch_fast_c<S, BITS, 5, XF16>(a, cus, s); break;
    case 6: if constexpr (XF16) launch_fast_c<S, BITS, 6, XF16>(a, cus, s); break;
    case 7: if constexpr (XF16) launch_fast_c<S, BITS, 7, XF16>(a, cus, s); break;
    default: if constexpr (XF16) launch_fast_c<S, BITS, 8, XF16>(a, cus, s); break;
  }
}

template <bool XF16>
static void launch_fast(const WView &w, const GemvArgs &a, int cus, hipStream_t s) {
  if (w.bits == 12) {
    if (w.S == 1) launch_fast_s<1, 12, XF16>(a, cus, s);
    else launch_fast_s<2, 12, XF16>(a, cus, s);
  } else {
    switch (w.S) {
      case 1: launch_fast_s<1, 8, XF16>(a, cus, s); break;
      case 2: launch_fast_s<2, 8, XF16>(a, cus, s); break;
      case 3: launch_fast_s<3, 8, XF16>(a, cus, s); break;
      default: launch_fast_s<4, 8, XF16>(a, cus, s); break;
    }
  }
}

template <int BITS>
static void launch_gen_bits(const WView &w, const GemvArgs &a, int xt, int cus, hipStream_t s) {
  const bool xl = w.k <= kGenMaxXLds;
  const bool g4 = (w.G % 4) == 0;
  int nwg = (a.n + kGenWaves - 1) / kGenWaves;
  if (nwg > cus * 2) nwg = cus * 2;
  if (g4 && xl) hipLaunchKernelGGL((k_gemv_gen<BITS, 4, true>), dim3(nwg), dim3(kGenWaves * 64), 0, s, a, xt);
  else if (g4) hipLaunchKernelGGL((k_gemv_gen<BITS, 4, false>), dim3(nwg), dim3(kGenWaves * 64), 0, s, a, xt);
  else if (xl) hipLaunchKernelGGL((k_gemv_gen<BITS, 1, true>), dim3(nwg), dim3(kGenWaves * 64), 0, s, a, xt);
  else hipLaunchKernelGGL((k_gemv_gen<BITS, 1, false>), dim3(nwg), dim3(kGenWaves * 64), 0, s, a, xt);
}

hipError_t launch_gemv_token(const WView &w, const void *x, int xt, float *y, hipStream_t s) {
  GemvArgs a = make_args(w);
  a.x = x;
  a.y = y;
  const int cus = device_cu_count();
  if (gemv_fast_eligible(w, xt)) {
    if (xt == VQ_BF16) launch_fast<true>(w, a, cus, s);
    else launch_fast<false>(w, a, cus, s);
  } else {
    if (w.bits == 8) launch_gen_bits<8>(w, a, xt, cus, s);
    else if (w.bits == 12) launch_gen_bits<12>(w, a, xt, cus, s);
    else launch_gen_bits<16>(w, a, xt, cus, s);
  }
  return hipGetLastError();
}

}  // namespace vqmm
