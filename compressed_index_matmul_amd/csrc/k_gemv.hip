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
template <int S, int BITS, int CPL, int WAVES, bool XF16, int RB>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_lds(GemvArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int CBN = S << BITS;                 // codebook rows of all stages
  constexpr int CB_ITERS = (CBN + NT - 1) / NT;  // 1 KiB LDS-direct loads per wave
  constexpr int XV = XF16 ? 4 : 8;               // 16-byte x vectors per chunk
  __shared__ uint4 s_cb[CBN];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int stride = gridDim.x * WAVES;
  int row = blockIdx.x * WAVES + wave;
  const int last = a.n - 1;

  // Global loads are issued oldest-first in the order they are needed:
  // codebooks, then x, then the first row's indices, so waiting for the
  // codebooks does not wait for anything else.  Chunks past the end of the
  // row load a valid duplicate and are masked out of the sum; no branch
  // surrounds a load, so every load stays in flight until its first use.
  // Codebooks stream straight into LDS (global_load_lds_dwordx4: lane l of a
  // wave writes 16 bytes at the wave's LDS base + 16 l), no registers used.
#pragma unroll
  for (int r = 0; r < CB_ITERS; ++r) {
    const int blk = (r * WAVES + wave) * 64;  // first codebook row of this wave's 1 KiB
    if (blk < CBN) {
      const uint4 *src = reinterpret_cast<const uint4 *>(a.cb[blk >> BITS]) + (blk & ((1 << BITS) - 1)) + lane;
      lds_direct_16(src, s_cb + blk);
    }
  }
  int cc[CPL];
  bool ok[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    ok[j] = c < a.C;
    cc[j] = ok[j] ? c : a.C - 1;
  }
  uint4 xr[CPL][XV];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const uint4 *px = XF16 ? reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.x) + 32 * cc[j])
                           : reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(a.x) + 32 * cc[j]);
#pragma unroll
    for (int v = 0; v < XV; ++v) xr[j][v] = px[v];
  }

  // Rows of this wave: row0 + k * stride.  They are processed in batches of
  // RB rows whose index loads are all in flight together; two register sets
  // alternate so the next batch loads while the current one is computed.
  // Guards are wave-uniform (a row exists or not for the whole wave).
  const int row0 = row;
  uint32_t L[RB][CPL][S], H[RB][CPL][S], SCb[RB][CPL];
#define VQ_LOAD_BATCH(B_, L_, H_, SC_)                                                     \
  _Pragma("unroll") for (int i = 0; i < RB; ++i) {                                         \
    const int rr = row0 + ((B_) * RB + i) * stride;                                        \
    if (rr < a.n) {                                                                        \
      const size_t rb = (size_t)rr * a.G;                                                  \
      _Pragma("unroll") for (int j = 0; j < CPL; ++j) {                                    \
        _Pragma("unroll") for (int t = 0; t < S; ++t) {                                    \
          L_[i][j][t] = *reinterpret_cast<const uint32_t *>(a.lo[t] + rb + 4 * cc[j]);     \
          if (BITS == 12)                                                                  \
            H_[i][j][t] = *reinterpret_cast<const uint16_t *>(a.hi[t] + (rb >> 1) + 2 * cc[j]); \
        }                                                                                  \
        SC_[i][j] = a.sc[(size_t)rr * a.nblk + (32 * cc[j]) / a.bs];                       \
      }                                                                                    \
    }                                                                                      \
  }
  VQ_LOAD_BATCH(0, L, H, SCb);

  // this lane's slice of x, held for the whole launch
  half2_t xh[XF16 ? CPL : 1][16];
  float xf[XF16 ? 1 : CPL][32];
  int xexp = 0;
  if (XF16) {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t w4[4] = {xr[j][v].x, xr[j][v].y, xr[j][v].z, xr[j][v].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float m2 = fmaxf(fabsf(bf2f(w4[e] & 0xffffu)), fabsf(bf2f(w4[e] >> 16)));
          mx = ok[j] ? fmaxf(mx, m2) : mx;
        }
      }
    // the largest |x| scaled into [2^14, 2^15): fp16 holds every bf16 value
    // within 2^28 of it exactly
    if (mx > 0.f) xexp = 14 - ilogbf(mx);
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t w4[4] = {xr[j][v].x, xr[j][v].y, xr[j][v].z, xr[j][v].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          xh[j][4 * v + e] = half2_t{(_Float16)ldexpf(bf2f(w4[e] & 0xffffu), xexp),
                                     (_Float16)ldexpf(bf2f(w4[e] >> 16), xexp)};
      }
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        xf[j][4 * v] = __uint_as_float(xr[j][v].x);
        xf[j][4 * v + 1] = __uint_as_float(xr[j][v].y);
        xf[j][4 * v + 2] = __uint_as_float(xr[j][v].z);
        xf[j][4 * v + 3] = __uint_as_float(xr[j][v].w);
      }
  }
  // the LDS-direct codebook loads of this wave have landed; then the barrier
  // makes every wave's part visible
  wait_all_memory();
  __syncthreads();

  // One row: gather every codebook row of a chunk first, then its dot
  // products; scale per chunk; masked chunks add nothing.
#define VQ_ROW(R_, L_, H_, SC_)                                                              \
  {                                                                                          \
    float acc = 0.f;                                                                         \
    _Pragma("unroll") for (int j = 0; j < CPL; ++j) {                                        \
      uint4 v[S][4];                                                                         \
      _Pragma("unroll") for (int t = 0; t < S; ++t)                                          \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                        \
        uint32_t idx = (L_[j][t] >> (8 * q)) & 0xffu;                                        \
        if (BITS == 12) idx |= ((H_[j][t] >> (4 * q)) & 0xfu) << 8;                          \
        v[t][q] = s_cb[(t << BITS) + idx];                                                   \
      }                                                                                      \
      float d = 0.f;                                                                         \
      _Pragma("unroll") for (int t = 0; t < S; ++t)                                          \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                        \
        if (XF16) {                                                                          \
          d = __builtin_amdgcn_fdot2(as_h2(v[t][q].x), xh[j][4 * q + 0], d, false);          \
          d = __builtin_amdgcn_fdot2(as_h2(v[t][q].y), xh[j][4 * q + 1], d, false);          \
          d = __builtin_amdgcn_fdot2(as_h2(v[t][q].z), xh[j][4 * q + 2], d, false);          \
          d = __builtin_amdgcn_fdot2(as_h2(v[t][q].w), xh[j][4 * q + 3], d, false);          \
        } else {                                                                             \
          const uint32_t hv[4] = {v[t][q].x, v[t][q].y, v[t][q].z, v[t][q].w};               \
          _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                    \
            d = fmaf(h2f(hv[e] & 0xffffu), xf[j][8 * q + 2 * e], d);                         \
            d = fmaf(h2f(hv[e] >> 16), xf[j][8 * q + 2 * e + 1], d);                         \
          }                                                                                  \
        }                                                                                    \
      }                                                                                      \
      acc = ok[j] ? fmaf(h2f(SC_[j]), d, acc) : acc;                                         \
    }                                                                                        \
    if (XF16) acc = ldexpf(acc, -xexp);                                                      \
    const float tot = wave_sum(acc);                                                         \
    if (lane == 0) a.y[R_] = tot;                                                            \
  }
#define VQ_BATCH(B_, L_, H_, SC_)                                                            \
  _Pragma("unroll") for (int i = 0; i < RB; ++i) {                                           \
    const int rr = row0 + ((B_) * RB + i) * stride;                                          \
    if (rr < a.n) VQ_ROW(rr, L_[i], H_[i], SC_[i]);                                          \
  }

  const int nrows = row0 < a.n ? (a.n - 1 - row0) / stride + 1 : 0;  // rows of this wave
  const int nbatch = (nrows + RB - 1) / RB;
  uint32_t L2[RB][CPL][S], H2[RB][CPL][S], SC2[RB][CPL];
  for (int b = 0; b < nbatch; b += 2) {
    if (b + 1 < nbatch) VQ_LOAD_BATCH(b + 1, L2, H2, SC2);
    VQ_BATCH(b, L, H, SCb);
    if (b + 1 >= nbatch) break;
    if (b + 2 < nbatch) VQ_LOAD_BATCH(b + 2, L, H, SCb);
    VQ_BATCH(b + 1, L2, H2, SC2);
  }
#undef VQ_BATCH
#undef VQ_ROW
#undef VQ_LOAD_BATCH
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

template <int S, int BITS, int CPL, int W, int RB, bool XF16>
static void launch_fast_w(const GemvArgs &a, int nwg, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv_lds<S, BITS, CPL, W, XF16, RB>), dim3(nwg), dim3(W * 64), 0, s, a);
}

// Persistent grid of one workgroup per CU slot (two when the codebooks take
// <= 80 KiB of LDS).  Waves per workgroup and rows in flight per wave (RB) are
// chosen so that the x slice, two batches of row indices and the gathers fit
// in the registers a wave gets: 16 waves -> 128 VGPRs, 8 -> 256, 4 -> 512.
template <int S, int BITS, int CPL, bool XF16>
static void launch_fast_c(const GemvArgs &a, int cus, hipStream_t s) {
  constexpr size_t lds = (size_t)(S << BITS) * 16;
  const int slots = cus * (lds > 81920 ? 1 : 2);
  constexpr int xload = CPL * (XF16 ? 1 : 2) * (S > 2 ? 2 : 1);
  auto grid = [&](int w) { const int g = (a.n + w - 1) / w; return g < slots ? g : slots; };
  auto rows_per_wave = [&](int w) { const int g = grid(w); return (a.n + g * w - 1) / (g * w); };
  if constexpr (xload <= 2) {
    if (rows_per_wave(16) <= 1) launch_fast_w<S, BITS, CPL, 16, 1, XF16>(a, grid(16), s);
    else launch_fast_w<S, BITS, CPL, 8, 4, XF16>(a, grid(8), s);
  } else if constexpr (xload <= 4) {
    if (rows_per_wave(8) <= 1) launch_fast_w<S, BITS, CPL, 8, 1, XF16>(a, grid(8), s);
    else launch_fast_w<S, BITS, CPL, 8, 2, XF16>(a, grid(8), s);
  } else {
    if (rows_per_wave(4) <= 1) launch_fast_w<S, BITS, CPL, 4, 1, XF16>(a, grid(4), s);
    else launch_fast_w<S, BITS, CPL, 4, 2, XF16>(a, grid(4), s);
  }
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
