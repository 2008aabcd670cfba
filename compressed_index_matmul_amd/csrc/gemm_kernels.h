// Kernel templates of the many-token product on matrix cores, shared by the
// translation units that instantiate them (k_gemm.hip: the plain formats;
// k_gemm_ladder.hip: mixed-width ladders and stage scales).
#pragma once

#include <type_traits>

#include "vqmm_device.h"
#include "vqmm_internal.h"

namespace vqmm {

struct GemmArgs {
  const uint8_t *lo[VQ_MAX_STAGES];
  const uint8_t *hi[VQ_MAX_STAGES];
  const uint16_t *i16[VQ_MAX_STAGES];
  const uint16_t *cb[VQ_MAX_STAGES];
  const uint16_t *sc;
  const uint16_t *x;  // bf16 [m][k]
  float *y;           // [m][n]
  int m, n, k, G, S, nblk, bs;
  int gshift;  // log2(scale_block / 8) when a power of two, else -1
  int tiles_m, tiles_n, per_xcd;
  uint64_t smagic;  // ceil(2^32 / (scale_block / 32)): K step -> scale block by a multiply
  int sb[VQ_MAX_STAGES];     // index width of each stage
  float rs[VQ_MAX_STAGES];   // stage scales
  int cboff[VQ_MAX_STAGES];  // first LDS codebook row of each stage (BITS = 0 kernels)
  int cbrows;                // codebook rows of all stages
  // fp16 path of the 256-token tile kernels (null xh: the bf16 path):
  const uint16_t *xh;  // x as fp16 in A-fragment order (k_x_f16), m_pad tokens
  const float *xf;     // [m_pad] per-token factors undoing the rescale of xh
  int m_pad;           // tokens rounded up to 16
};

// LDS codebook rows of the BITS = 0 (per-stage widths) kernels: 128 KiB.
constexpr int kLadderCbRows = 8192;

// Copy the codebooks of a ladder of per-stage widths into LDS, stage t from
// row a.cboff[t] (plain loads; the caller synchronises).
__device__ __forceinline__ void stage_ladder_codebooks(const GemmArgs &a, uint4 *s_cb, int tid, int nthreads) {
  // stage pointers selected among values, not indexed (a per-thread index
  // into the argument array would be a vector load per element)
  const uint4 *cb[VQ_MAX_STAGES];
#pragma unroll
  for (int t = 0; t < VQ_MAX_STAGES; ++t) cb[t] = static_cast<const uint4 *>(uniform_ptr(a.cb[t < a.S ? t : 0]));
  for (int i = tid; i < a.cbrows; i += nthreads) {
    const bool s1 = a.S > 1 && i >= a.cboff[1], s2 = a.S > 2 && i >= a.cboff[2], s3 = a.S > 3 && i >= a.cboff[3];
    const uint4 *p = s3 ? cb[3] : s2 ? cb[2] : s1 ? cb[1] : cb[0];
    const int off = s3 ? a.cboff[3] : s2 ? a.cboff[2] : s1 ? a.cboff[1] : 0;
    s_cb[i] = p[i - off];
  }
}

// Scale block of group g (8 columns): g / (scale_block / 8).
__device__ __forceinline__ int scale_blk(const GemmArgs &a, int g) {
  return a.gshift >= 0 ? (g >> a.gshift) : (8 * g) / a.bs;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Decode group g of W row `row` to 8 fp32 weights: stage sum and scale in
// fp32 (summation starts from stage 0).  BITS = 0: per-stage widths (a.sb),
// each entry times its stage scale.
template <int S, int BITS, bool CB_LDS>
__device__ __forceinline__ void decode_group_f32(const GemmArgs &a, const uint4 *s_cb, int row, int g, float (&w)[8]) {
  const size_t f = (size_t)row * a.G + g;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const uint32_t idx = load_index(BITS ? BITS : a.sb[t], a.lo[t], a.hi[t], a.i16[t], f);
    const uint4 v = CB_LDS ? s_cb[(BITS ? (t << BITS) : a.cboff[t]) + idx] : reinterpret_cast<const uint4 *>(a.cb[t])[idx];
    const uint32_t hv[4] = {v.x, v.y, v.z, v.w};
    const float r = BITS ? 1.f : a.rs[t];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float c0 = h2f(hv[e] & 0xffffu), c1 = h2f(hv[e] >> 16);
      if (BITS == 0) {
        c0 *= r;
        c1 *= r;
      }
      w[2 * e] = (t == 0) ? c0 : w[2 * e] + c0;
      w[2 * e + 1] = (t == 0) ? c1 : w[2 * e + 1] + c1;
    }
  }
  const float s = h2f(a.sc[(size_t)row * a.nblk + (8 * g) / a.bs]);
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] *= s;
}

// The same group as 8 bf16 (packed in a uint4).
template <int S, int BITS, bool CB_LDS>
__device__ __forceinline__ uint4 decode_group_bf16(const GemmArgs &a, const uint4 *s_cb, int row, int g) {
  float w[8];
  decode_group_f32<S, BITS, CB_LDS>(a, s_cb, row, g, w);
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = f2bf(w[2 * e]) | (f2bf(w[2 * e + 1]) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// large M
// ---------------------------------------------------------------------------
constexpr int kLM = 256, kLN = 128;
constexpr int kWP = 40;  // bf16 per W-tile row in LDS: 32 + 8 pad (80 B rows: conflict-free b128)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// fp32 sum of two fp16 values taken from the low (HI=false) or high halves
// of a and b, rounded once (v_fma_mix_f32: a * 1.0 + b with both sources
// read as fp16).
template <bool HI>
__device__ __forceinline__ float add_f16(uint32_t a, uint32_t b) {
  float d;
#if defined(__HIP_DEVICE_COMPILE__)
  if (HI)
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(a), "v"(b));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,1]" : "=v"(d) : "v"(a), "v"(b));
#else
  d = h2f(HI ? a >> 16 : a & 0xffffu) + h2f(HI ? b >> 16 : b & 0xffffu);
#endif
  return d;
}

// 8 fp32 weights as two bf16 parts for the few-token products: hi = w
// rounded to bf16, lo = (w - hi) rounded to bf16.  w - hi is exact in fp32
// (at most 16 significant bits).  For w in [2^e, 2^(e+1)), |w - hi| <=
// 2^(e-8), and below that bound its bf16 rounding is off by at most
// 2^(e-17) (at the bound it is a power of two, exact), so |w - (hi + lo)| <=
// 2^-17 |w|, where hi alone is off by up to 2^-8 |w|; two bf16 MFMAs (x hi,
// then x lo) then give every output about the accuracy of exact fp16
// products.
__device__ __forceinline__ void split_bf16(const float (&w)[8], uint4 &hi, uint4 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_bf16(w[2 * e], w[2 * e + 1]);
    l[e] = pack_bf16(w[2 * e] - __uint_as_float(h[e] << 16), w[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// 8 weights of one group in fp32: sum of the stage vectors (each partial sum
// rounded once), times the scale.
template <int S>
__device__ __forceinline__ void group_to_f32(const uint4 (&v)[S], float sf, float (&w)[8]) {
  const uint32_t h0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
  if (S == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[2 * e] = h2f(h0[e] & 0xffffu);
      w[2 * e + 1] = h2f(h0[e] >> 16);
    }
  } else {
    const uint32_t h1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[2 * e] = add_f16<false>(h0[e], h1[e]);
      w[2 * e + 1] = add_f16<true>(h0[e], h1[e]);
    }
#pragma unroll
    for (int t = 2; t < S; ++t) {
      const uint32_t ht[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[2 * e] += h2f(ht[e] & 0xffffu);
        w[2 * e + 1] += h2f(ht[e] >> 16);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] *= sf;
}

// The same rounded to bf16.
template <int S>
__device__ __forceinline__ uint4 group_to_bf16(const uint4 (&v)[S], float sf) {
  float w[8];
  group_to_f32<S>(v, sf, w);
  return make_uint4(pack_bf16(w[0], w[1]), pack_bf16(w[2], w[3]), pack_bf16(w[4], w[5]), pack_bf16(w[6], w[7]));
}

// 8 weights of one group in fp32 with stage scales: sum of each stage vector
// times its scale (from stage 0), times the block scale.
template <int S>
__device__ __forceinline__ void group_to_f32_scaled(const uint4 (&v)[S], float sf, const float *rs, float (&w)[8]) {
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const uint32_t ht[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c0 = h2f(ht[e] & 0xffffu) * rs[t], c1 = h2f(ht[e] >> 16) * rs[t];
      w[2 * e] = t == 0 ? c0 : w[2 * e] + c0;
      w[2 * e + 1] = t == 0 ? c1 : w[2 * e + 1] + c1;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] *= sf;
}

// The same rounded to bf16.
template <int S>
__device__ __forceinline__ uint4 group_to_bf16_scaled(const uint4 (&v)[S], float sf, const float *rs) {
  float w[8];
  group_to_f32_scaled<S>(v, sf, rs, w);
  return make_uint4(pack_bf16(w[0], w[1]), pack_bf16(w[2], w[3]), pack_bf16(w[4], w[5]), pack_bf16(w[6], w[7]));
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// 8 weights of one group as fp16 for the fp16 matrix-core path: c0 s with
// one stage, (c0 + c1) s with two, in packed-half arithmetic (v_pk_add_f16,
// v_pk_mul_f16), each operation rounded once to nearest even.  The sum is
// rounded relative to itself and then the product, so |w16 - w| <= (2^-10 +
// 2^-22) |w| for every weight (subnormal results aside: absolute error at
// most 2^-25), where bf16 weights carry up to 2^-8 |w|.  sc16: fp16 bits of
// the block scale.
template <int S>
__device__ __forceinline__ uint4 group_to_f16(const uint4 (&v)[S], uint32_t sc16) {
  static_assert(S == 1 || S == 2, "one or two stages");
  const half2_t s2 = as_h2(sc16 | (sc16 << 16));
  auto pair = [&](uint32_t c0, uint32_t c1) -> uint32_t {
    const half2_t w = S == 1 ? as_h2(c0) : as_h2(c0) + as_h2(c1);
    return __builtin_bit_cast(uint32_t, w * s2);
  };
  return make_uint4(pair(v[0].x, v[S - 1].x), pair(v[0].y, v[S - 1].y), pair(v[0].z, v[S - 1].z),
                    pair(v[0].w, v[S - 1].w));
}

// The same with stage scales: s sum_t r_t c_t in fp32 (summation from stage
// 0), rounded once to fp16.
template <int S>
__device__ __forceinline__ uint4 group_to_f16_scaled(const uint4 (&v)[S], float sf, const float *rs) {
  float w[8];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const uint32_t ht[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c0 = h2f(ht[e] & 0xffffu) * rs[t], c1 = h2f(ht[e] >> 16) * rs[t];
      w[2 * e] = t == 0 ? c0 : w[2 * e] + c0;
      w[2 * e + 1] = t == 0 ? c1 : w[2 * e + 1] + c1;
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)(sf * w[2 * e]), (_Float16)(sf * w[2 * e + 1])});
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Everything one thread needs from global memory for one K step (4 groups,
// 32 columns) of the large-M kernel: index bits of its two groups for every
// stage, their scales, and the wave's A fragments (x) for the step.
template <int S>
struct StepRegs {
  uint32_t lo[S];   // 8/12-bit: 2 low bytes; 16-bit: two indices
  uint32_t hi[S];   // 12-bit: one byte = two nibbles
  uint32_t sc[2];   // fp16 bits of the two groups' scales
  uint4 av[2][2];   // A fragments [kk][i]
};

// Per-lane constant parts of every address of the large-M kernel (32-bit
// element offsets); the K step adds a wave-uniform part, so each load is a
// scalar base plus a 32-bit lane offset and costs no vector address math.
struct LaneOffsets {
  uint32_t f;       // flat group index of the thread's first group at step 0
  uint32_t scrow;   // first scale of the thread's W row
  uint32_t a[2];    // x byte offset of the lane's A rows (plus its k half)
  int kh;           // the lane's k half within a 16-column MFMA step: 0 or 8
};

// A 16-byte load from a wave-uniform base plus a 32-bit lane byte offset.
__device__ __forceinline__ uint4 ld16(const void *base, uint32_t off) {
  return *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(base) + off);
}

template <int S, int BITS, bool ALIGNED>
__device__ __forceinline__ void gemm_load_step(const GemmArgs &a, int ks, int dg, const LaneOffsets &o,
                                               StepRegs<S> &R) {
  const int g0 = ks * 4 + dg;  // first of this thread's two groups
  if (ALIGNED) {
#pragma unroll
    for (int t = 0; t < S; ++t) {
      if (BITS == 16) {
        R.lo[t] = *reinterpret_cast<const uint32_t *>(a.i16[t] + 4 * ks + o.f);
      } else {
        R.lo[t] = *reinterpret_cast<const uint16_t *>(a.lo[t] + 4 * ks + o.f);
        if (BITS == 12) R.hi[t] = (a.hi[t] + 2 * ks)[o.f >> 1];
      }
    }
    R.sc[0] = a.sc[o.scrow + scale_blk(a, g0)];
    R.sc[1] = a.sc[o.scrow + scale_blk(a, g0 + 1)];
  } else {
    const size_t f = (size_t)o.f + 4 * ks;
#pragma unroll
    for (int t = 0; t < S; ++t) {
      uint32_t i0 = 0, i1 = 0;
      const int bt = BITS ? BITS : a.sb[t];
      if (g0 < a.G) i0 = load_index(bt, a.lo[t], a.hi[t], a.i16[t], f);
      if (g0 + 1 < a.G) i1 = load_index(bt, a.lo[t], a.hi[t], a.i16[t], f + 1);
      R.lo[t] = i0 | (i1 << 16);  // unpacked form for the ragged path
    }
    R.sc[0] = g0 < a.G ? a.sc[o.scrow + scale_blk(a, g0)] : 0;
    R.sc[1] = g0 + 1 < a.G ? a.sc[o.scrow + scale_blk(a, g0 + 1)] : 0;
  }
  const uint16_t *xs = a.x + 32 * ks;  // wave-uniform
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    // column of the load: 32 ks + 16 kk + the lane's k half (o.a includes it)
    const bool in = ALIGNED || 32 * ks + 16 * kk + o.kh < a.k;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      R.av[kk][i] = in ? ld16(xs + 16 * kk, o.a[i]) : make_uint4(0, 0, 0, 0);
  }
}

// Buffer descriptors and per-lane offsets of the aligned large-M kernel
// (K % 32 == 0, scale_block % 32 == 0): every load of a K step is a scalar
// descriptor plus a constant lane offset plus a wave-uniform step offset.
template <int S>
struct BufSet {
  buf_t lo[S], hi[S], sc, x;
  uint32_t vlo, vhi, vsc, va[2];
};

template <int S, int BITS>
__device__ __forceinline__ void gemm_bufs(const GemmArgs &a, int wrow_c, int dg, const LaneOffsets &o, BufSet<S> &B) {
  const uint32_t ng = (uint32_t)a.n * a.G;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    B.lo[t] = BITS == 16 ? make_buf(a.i16[t], 2 * ng) : make_buf(a.lo[t], ng);
    B.hi[t] = make_buf(BITS == 12 ? a.hi[t] : a.lo[t], BITS == 12 ? (ng + 1) / 2 : ng);
  }
  B.sc = make_buf(a.sc, 2u * a.n * a.nblk);
  B.x = make_buf(a.x, 2u * a.m * a.k);
  const uint32_t f = (uint32_t)wrow_c * a.G + dg;
  B.vlo = (BITS == 16 ? 2 : 1) * f;
  B.vhi = f >> 1;  // f is even: G % 4 == 0 and dg is 0 or 2
  B.vsc = 2u * wrow_c * a.nblk;
  B.va[0] = o.a[0];
  B.va[1] = o.a[1];
}

template <int S, int BITS>
__device__ __forceinline__ void gemm_load_step_buf(const GemmArgs &a, const BufSet<S> &B, int ks, StepRegs<S> &R) {
#pragma unroll
  for (int t = 0; t < S; ++t) {
    if (BITS == 16) {
      R.lo[t] = buf_u32(B.lo[t], B.vlo, 8u * ks);
    } else {
      R.lo[t] = buf_u16(B.lo[t], B.vlo, 4u * ks);
      if (BITS == 12) R.hi[t] = buf_u8(B.hi[t], B.vhi, 2u * ks);
    }
  }
  const uint32_t blk = (uint32_t)(((uint64_t)ks * a.smagic) >> 32);  // (32 ks) / scale_block
  R.sc[0] = buf_u16(B.sc, B.vsc, 2u * blk);
  R.sc[1] = R.sc[0];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 2; ++i) R.av[kk][i] = buf_u128(B.x, B.va[i], 64u * ks + 32u * kk);
}

// Decode the thread's two groups of step ks into the LDS W tile.
template <int S, int BITS, bool CB_LDS, bool ALIGNED>
__device__ __forceinline__ void gemm_decode_store(const GemmArgs &a, const uint4 *s_cb, const StepRegs<S> &R,
                                                  int ks, int dg, bool wok, uint16_t *wt, int drow) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int g = ks * 4 + dg + u;
    uint4 v[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
      uint32_t idx;
      if (!ALIGNED || BITS == 16) idx = (R.lo[t] >> (16 * u)) & 0xffffu;
      else {
        idx = (R.lo[t] >> (8 * u)) & 0xffu;
        if (BITS == 12) idx |= ((R.hi[t] >> (4 * u)) & 0xfu) << 8;
      }
      v[t] = CB_LDS ? s_cb[(BITS ? (t << BITS) : a.cboff[t]) + idx] : reinterpret_cast<const uint4 *>(a.cb[t])[idx];
    }
    uint4 pk = group_to_bf16<S>(v, h2f(R.sc[u]));
    if (!wok || (!ALIGNED && g >= a.G)) pk = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(&wt[drow * kWP + 8 * (dg + u)]) = pk;
  }
}

// Tile 256 x 128, K step 32, 4 waves stacked along M, each owning 64 token
// rows x all 128 W columns as 2 x 4 accumulator blocks of
// v_mfma_f32_32x32x16_bf16 (x fragments are never loaded twice).  Every
// thread decodes two groups per K step (LDS codebook gathers, fp32 stage sum
// and scale, bf16) into one of two LDS W tiles.  Software pipeline, one
// barrier per step: iteration k reads the B fragments of tile k, issues the
// codebook gathers of step k+1, then interleaves the 16 MFMAs of step k with
// the decode of step k+1 into the other tile.  Global loads (indices,
// scales, x fragments) run four steps ahead in a ring of four register sets.
template <int S, int BITS, bool CB_LDS, bool ALIGNED>
__global__ __launch_bounds__(256) void k_gemm_large(GemmArgs a) {
  __shared__ uint4 s_cb[CB_LDS ? (BITS ? (S << BITS) : kLadderCbRows) : 1];
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][kLN * kWP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int L = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  if (L >= a.tiles_m * a.tiles_n) return;  // whole workgroup, before any barrier
  const int m0 = (L / a.tiles_n) * kLM;
  const int n0 = (L % a.tiles_n) * kLN;

  if (CB_LDS) {
    if constexpr (BITS != 0) {
      constexpr int CBN = S << BITS;
#pragma unroll 4
      for (int r = 0; r < CBN / 256; ++r) {
        const int blk = (r * 4 + wave) * 64;
        lds_direct_16(reinterpret_cast<const uint4 *>(a.cb[blk >> BITS]) + (blk & ((1 << BITS) - 1)) + lane,
                      s_cb + blk);
      }
    } else {
      stage_ladder_codebooks(a, s_cb, tid, 256);  // visible after the barrier below
    }
  }
  const int drow = tid >> 1;     // W-tile row decoded by this thread
  const int dg = 2 * (tid & 1);  // first of its two groups in a K step
  const int wrow = n0 + drow;
  const bool wok = wrow < a.n;
  const int wrow_c = wok ? wrow : a.n - 1;  // loads stay in bounds; result zeroed
  LaneOffsets o;
  o.f = (uint32_t)wrow_c * a.G + dg;
  o.scrow = (uint32_t)wrow_c * a.nblk;
  o.kh = 8 * (lane >> 5);
  // A rows of this lane (one per 32-row block).  Rows past m load row m-1:
  // they only feed output rows past m, which are never stored.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int r = m0 + wave * 64 + 32 * i + (lane & 31);
    r = r < a.m ? r : a.m - 1;
    o.a[i] = 2u * ((uint32_t)r * a.k + o.kh);
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nks = (a.G + 3) / 4;
  StepRegs<S> R0, R1, R2, R3;
  BufSet<S> B;
  if (ALIGNED) gemm_bufs<S, BITS>(a, wrow_c, dg, o, B);
  // Unconditional prefetch (past the last step it reloads the last step):
  // with no branch around the loads the wait counts stay exact.
  auto load = [&](int ks, StepRegs<S> &R) {
    if (ALIGNED) gemm_load_step_buf<S, BITS>(a, B, ks < nks ? ks : nks - 1, R);
    else gemm_load_step<S, BITS, ALIGNED>(a, ks < nks ? ks : nks - 1, dg, o, R);
  };
  // codebook gathers of the thread's two groups of a step
  auto gather = [&](const StepRegs<S> &R, uint4 (&v)[2][S]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < S; ++t) {
        uint32_t idx;
        if (!ALIGNED || BITS == 16) idx = (R.lo[t] >> (16 * u)) & 0xffffu;
        else {
          idx = (R.lo[t] >> (8 * u)) & 0xffu;
          if (BITS == 12) idx |= ((R.hi[t] >> (4 * u)) & 0xfu) << 8;
        }
        v[u][t] = CB_LDS ? s_cb[(BITS ? (t << BITS) : a.cboff[t]) + idx] : reinterpret_cast<const uint4 *>(a.cb[t])[idx];
      }
  };
  // decode group u of step ks (gathered vectors v) and store it in tile wt
  // (aligned path: W rows past n only feed output columns that are never
  // stored, so they are decoded from the clamped row and not zeroed)
  auto decode = [&](int ks, int u, const StepRegs<S> &R, const uint4 (&v)[S], uint16_t *wt) {
    const float sf = h2f(R.sc[ALIGNED ? 0 : u]);
    uint4 pk = BITS ? group_to_bf16<S>(v, sf) : group_to_bf16_scaled<S>(v, sf, a.rs);
    const int g = ks * 4 + dg + u;
    if (!ALIGNED && (!wok || g >= a.G)) pk = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(&wt[drow * kWP + 8 * (dg + u)]) = pk;
  };
  auto mma4 = [&](const StepRegs<S> &R, const bf16x8_t (&bfr)[2][4], int kk, int i) {
    const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, R.av[kk][i]);
#pragma unroll
    for (int jn = 0; jn < 4; ++jn)
      acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bfr[kk][jn], acc[i][jn], 0, 0, 0);
  };
  // Iteration ks: MFMAs of step ks (A fragments in Rm, B fragments from tile
  // ks & 1) with the decode of step ks+1 (indices in Rd) into the other
  // tile, then the loads of step ks+4 into Rm, then the barrier.  The tile
  // written here was last read in iteration ks-1, before its barrier.
  auto iter = [&](int ks, StepRegs<S> &Rm, const StepRegs<S> &Rd) {
    const uint16_t *wr = s_w[ks & 1];
    uint16_t *ww = s_w[(ks + 1) & 1];
    bf16x8_t bfr[2][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        bfr[kk][jn] = *reinterpret_cast<const bf16x8_t *>(&wr[(32 * jn + (lane & 31)) * kWP + 16 * kk + 8 * (lane >> 5)]);
    uint4 v[2][S];
    gather(Rd, v);
    sched_fence();
    mma4(Rm, bfr, 0, 0);
    sched_fence();
    decode(ks + 1, 0, Rd, v[0], ww);
    sched_fence();
    mma4(Rm, bfr, 0, 1);
    sched_fence();
    decode(ks + 1, 1, Rd, v[1], ww);
    sched_fence();
    mma4(Rm, bfr, 1, 0);
    sched_fence();
    mma4(Rm, bfr, 1, 1);
    sched_fence();
    load(ks + 4, Rm);
    __syncthreads();
  };

  load(0, R0);
  load(1, R1);
  load(2, R2);
  load(3, R3);
  wait_all_memory();  // codebook (LDS-direct) has landed (and the first steps)
  __syncthreads();
  {
    uint4 v[2][S];
    gather(R0, v);
    decode(0, 0, R0, v[0], s_w[0]);
    decode(0, 1, R0, v[1], s_w[0]);
  }
  __syncthreads();
  // main loop: four iterations per trip, a single exit (a loop with several
  // exits made the compiler move the accumulators between register files)
  int ks = 0;
  for (; ks + 4 <= nks; ks += 4) {
    iter(ks, R0, R1);
    iter(ks + 1, R1, R2);
    iter(ks + 2, R2, R3);
    iter(ks + 3, R3, R0);
  }
  // remainder: sets R0, R1, R2 hold steps ks, ks+1, ks+2
  const int rem = nks - ks;
  if (rem > 0) iter(ks, R0, R1);
  if (rem > 1) iter(ks + 1, R1, R2);
  if (rem > 2) iter(ks + 2, R2, R3);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int col = n0 + 32 * jn + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wave * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < a.m && col < a.n) a.y[(size_t)row * a.n + col] = acc[i][jn][r];
      }
    }
}

// ---------------------------------------------------------------------------
// large M, K % 256 == 0
// ---------------------------------------------------------------------------
// Index planes of one thread's W row for 4 K steps (16 groups): 16 low bytes
// and, for 12-bit indices, 16 high nibbles per stage.
template <int S>
struct Quad {
  uint4 lo[S];
  uint2 hi[S];
};

// x fragments (4 blocks of 16 tokens) and the thread's scale for one K step.
struct XStep {
  uint4 av[4];
  uint32_t sc;
};

// fp16 path: multiply each accumulator by its token's factor (the inverse
// of the power-of-two rescale of that token's x), acc[i][j][r] belonging to
// token m0 + 64 wave + 16 i + 4 (lane / 16) + r.
template <int NJ>
__device__ __forceinline__ void token_factors(const GemmArgs &a, int m0, int wave, int lane, f32x4 (&acc)[4][NJ]) {
  const buf_t bf = make_buf(a.xf, 4u * (uint32_t)a.m_pad);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t tok = (uint32_t)min(m0 + wave * 64 + 16 * i + 4 * (lane >> 4) + r, a.m_pad - 1);
      const float f = __uint_as_float(buf_u32(bf, 4u * tok, 0));
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j][r] *= f;
    }
}

// Tile 256 (tokens) x 128 (W rows), K step 32, 4 waves stacked along the
// tokens, each owning 64 x 128 as 4 x 8 blocks of v_mfma_f32_16x16x32_bf16
// (lane l of an A fragment holds 8 consecutive k of token l % 16, so each x
// load reads 64 contiguous bytes per token).  Every load is a buffer load:
// the index planes of 4 K steps at once (16 B + 8 B per stage and thread),
// x fragments and the scale per step.  Software pipeline over a ring of three
// LDS W tiles, one barrier per step: iteration k issues the codebook gathers
// of step k+2 and the B-fragment reads of step k+1 (published by the previous
// barrier), interleaves the 32 MFMAs of step k (B fragments read one
// iteration earlier) with the decode of step k+2, loads step k+4, then the
// barrier.  The tile written in iteration k holds step k-1, whose fragments
// were read in iteration k-2.
template <class LD, bool RS, bool F16 = false>
__global__ __launch_bounds__(256) void k_gemm_tile(GemmArgs a) {
  constexpr int S = LD::S;
  using frag_t = typename std::conditional<F16, f16x8_t, bf16x8_t>::type;
  __shared__ uint4 s_cb[LD::kRows];
  __shared__ __attribute__((aligned(16))) uint16_t s_w[3][kLN * kWP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int L = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  if (L >= a.tiles_m * a.tiles_n) return;  // whole workgroup, before any barrier
  const int m0 = (L / a.tiles_n) * kLM;
  const int n0 = (L % a.tiles_n) * kLN;
  if constexpr (LD::kUniform) {
    constexpr int BITS = LD::bits(0);
    constexpr int CBN = S << BITS;
#pragma unroll 4
    for (int r = 0; r < CBN / 256; ++r) {
      const int blk = (r * 4 + wave) * 64;
      lds_direct_16(reinterpret_cast<const uint4 *>(a.cb[blk >> BITS]) + (blk & ((1 << BITS) - 1)) + lane,
                    s_cb + blk);
    }
  } else {
    stage_ladder_lds<LD, 4>(a.cb, s_cb, wave, lane);
  }
  const int drow = tid >> 1;     // W-tile row decoded by this thread
  const int dg = 2 * (tid & 1);  // first of its two groups in a K step
  // W rows past n are decoded from the last row: they only feed output
  // columns past n, which are never stored
  const int wrow_c = min(n0 + drow, a.n - 1);
  const uint32_t ng = (uint32_t)a.n * a.G;
  buf_t blo[S], bhi[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    blo[t] = make_buf(LD::lo(t) ? a.lo[t] : a.hi[t], ng);
    bhi[t] = make_buf(LD::hi(t) ? a.hi[t] : a.lo[t], LD::hi(t) ? (ng + 1) / 2 : ng);
  }
  const buf_t bsc = make_buf(a.sc, 2u * a.n * a.nblk);
  const buf_t bx = F16 ? make_buf(a.xh, 2u * (uint32_t)a.m_pad * (uint32_t)a.k) : make_buf(a.x, 2u * a.m * a.k);
  const uint32_t vlo = (uint32_t)wrow_c * a.G;  // + 16 per quad
  const uint32_t vhi = vlo >> 1;                // + 8 per quad (G is even)
  const uint32_t vsc = 2u * wrow_c * a.nblk;
  // x byte offsets of this lane's token (one per 16-token block) and k chunk;
  // tokens past m load token m-1 and feed rows that are never stored
  // (fp16 path: the lane's 16 bytes of its token block's 1 KiB fragment
  // per K step; blocks past m_pad load the last one)
  uint32_t va[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (F16) {
      const uint32_t tb = (uint32_t)min(m0 + wave * 64 + 16 * i, a.m_pad - 16) / 16u;
      va[i] = 16u * (tb * (uint32_t)(a.k / 32) * 64u + (uint32_t)lane);
    } else {
      const int r = min(m0 + wave * 64 + 16 * i + (lane & 15), a.m - 1);
      va[i] = 2u * ((uint32_t)r * a.k + 8 * (lane >> 4));
    }
  }

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = a.G / 4;  // K steps (a multiple of 8)
  const int nq = a.G / 16;  // quads
  // Unconditional loads (past the end they reload the last step or quad):
  // no branch around a load, so the wait counts stay exact.
  auto load_quad = [&](int j, Quad<S> &Q) {
    j = min(j, nq - 1);
#pragma unroll
    for (int t = 0; t < S; ++t) {
      if (LD::lo(t)) Q.lo[t] = buf_u128(blo[t], vlo, 16u * j);
      if (LD::hi(t)) Q.hi[t] = buf_u64(bhi[t], vhi, 8u * j);
    }
  };
  auto load_x = [&](int ks, XStep &X) {
    ks = min(ks, nks - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) X.av[i] = buf_u128(bx, va[i], (F16 ? 1024u : 64u) * ks);
    const uint32_t blk = (uint32_t)(((uint64_t)ks * a.smagic) >> 32);  // (32 ks) / scale_block
    X.sc = buf_u16(bsc, vsc, 2u * blk);
  };
  // index of group u (0, 1) of the thread's pair in step s (0..3) of a quad
  auto idx_of = [&](const Quad<S> &Q, int s, int u, int t) -> uint32_t {
    uint32_t idx = 0;
    if (LD::lo(t)) {
      const uint32_t lw = s == 0 ? Q.lo[t].x : s == 1 ? Q.lo[t].y : s == 2 ? Q.lo[t].z : Q.lo[t].w;
      idx = (lw >> (8 * (dg + u))) & 0xffu;
    }
    if (LD::hi(t)) {
      const uint32_t hw = s < 2 ? Q.hi[t].x : Q.hi[t].y;  // nibbles of groups 8 (s / 2) .. + 7
      idx |= ((hw >> (4 * (4 * (s & 1) + dg + u))) & 0xfu) << LD::hshift(t);
    }
    return idx;
  };
  auto gather = [&](const Quad<S> &Q, int s, uint4 (&v)[2][S]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < S; ++t) v[u][t] = s_cb[LD::off(t) + idx_of(Q, s, u, t)];
  };
  auto decode = [&](int u, const uint4 (&v)[S], uint32_t sc, uint16_t *wt) {
    uint4 pk;
    if constexpr (F16) pk = RS ? group_to_f16_scaled<S>(v, h2f(sc), a.rs) : group_to_f16<S>(v, sc);
    else pk = RS ? group_to_bf16_scaled<S>(v, h2f(sc), a.rs) : group_to_bf16<S>(v, h2f(sc));
    *reinterpret_cast<uint4 *>(&wt[drow * kWP + 8 * (dg + u)]) = pk;
  };
  auto read_b = [&](const uint16_t *wr, frag_t (&bfr)[8]) {
#pragma unroll
    for (int jn = 0; jn < 8; ++jn)
      bfr[jn] = *reinterpret_cast<const frag_t *>(&wr[(16 * jn + (lane & 15)) * kWP + 8 * (lane >> 4)]);
  };
  auto mma8 = [&](const XStep &X, const frag_t (&bfr)[8], int i) {
    const frag_t afr = __builtin_bit_cast(frag_t, X.av[i]);
#pragma unroll
    for (int jn = 0; jn < 8; ++jn) {
      if constexpr (F16) acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr[jn], acc[i][jn], 0, 0, 0);
      else acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[jn], acc[i][jn], 0, 0, 0);
    }
  };
  // Iteration ks: B fragments of step ks+1 into Bn (tile (ks+1) % 3), MFMAs
  // of step ks (Xm, Bc), decode of step ks+2 (codebook vectors in v, gathered
  // one iteration earlier; scale in Xd) into tile (ks+2) % 3, gathers of step
  // ks+3 (quad Qg, step sg) into v, loads of step ks+4 into Xm (and, when
  // ks % 4 == 2, of quad (ks+6)/4 into Qn), barrier.
  auto iter = [&](int ks, XStep &Xm, const XStep &Xd, const frag_t (&Bc)[8], frag_t (&Bn)[8],
                  const Quad<S> &Qg, int sg, Quad<S> &Qn, bool quad_load, uint4 (&v)[2][S]) {
    uint16_t *ww = s_w[(ks + 2) % 3];
    read_b(s_w[(ks + 1) % 3], Bn);
    sched_fence();
    // 32 MFMAs with the decode's vector work between them: one MFMA, then
    // two VALU instructions, so the matrix core and the VALU run together
    mma8(Xm, Bc, 0);
    decode(0, v[0], Xd.sc, ww);
    mma8(Xm, Bc, 1);
    decode(1, v[1], Xd.sc, ww);
    gather(Qg, sg, v);
    mma8(Xm, Bc, 2);
    mma8(Xm, Bc, 3);
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      sched_group<0x008, 1>();
      sched_group<0x002, 2>();
    }
    sched_fence();
    load_x(ks + 4, Xm);  // before the index quad: see k_gemm_wide
    if (quad_load) load_quad((ks + 6) / 4, Qn);
    __syncthreads();
  };

  Quad<S> Q0, Q1;
  XStep X0, X1, X2, X3;
  load_quad(0, Q0);
  load_quad(1, Q1);
  load_x(0, X0);
  load_x(1, X1);
  load_x(2, X2);
  load_x(3, X3);
  wait_all_memory();  // codebook (LDS-direct) has landed (and the first steps)
  __syncthreads();
  uint4 v[2][S];
  gather(Q0, 0, v);
  decode(0, v[0], X0.sc, s_w[0]);
  decode(1, v[1], X0.sc, s_w[0]);
  gather(Q0, 1, v);
  decode(0, v[0], X1.sc, s_w[1]);
  decode(1, v[1], X1.sc, s_w[1]);
  gather(Q0, 2, v);  // step 2, decoded in iteration 0
  __syncthreads();
  frag_t B0[8], B1[8];
  read_b(s_w[0], B0);
  // eight steps (two quads) per trip; the three W tiles rotate with ks % 3
  // (compile-time inside the trip only when 3 divides the trip length, so the
  // tile index is computed at run time); quads alternate between Q0 and Q1
  for (int ks = 0; ks < nks; ks += 8) {
    // iteration ks+i gathers step ks+i+3: Q0 is last read in iteration ks
    // and refilled in ks+2 (first read in ks+5); Q1 is last read in ks+4
    // and refilled in ks+6 (first read in ks+9)
    iter(ks + 0, X0, X2, B0, B1, Q0, 3, Q1, false, v);
    iter(ks + 1, X1, X3, B1, B0, Q1, 0, Q1, false, v);
    iter(ks + 2, X2, X0, B0, B1, Q1, 1, Q0, true, v);   // quad (ks+8)/4 -> Q0
    iter(ks + 3, X3, X1, B1, B0, Q1, 2, Q0, false, v);
    iter(ks + 4, X0, X2, B0, B1, Q1, 3, Q0, false, v);
    iter(ks + 5, X1, X3, B1, B0, Q0, 0, Q1, false, v);
    iter(ks + 6, X2, X0, B0, B1, Q0, 1, Q1, true, v);   // quad (ks+12)/4 -> Q1
    iter(ks + 7, X3, X1, B1, B0, Q0, 2, Q1, false, v);
  }
  if constexpr (F16) token_factors(a, m0, wave, lane, acc);
  // tiles wholly inside y: descriptor stores as in the wide kernel
  if (m0 + kLM <= a.m && n0 + kLN <= a.n && (uint64_t)kLM * a.n * 4 < (1u << 31)) {
    const buf_t by = make_buf(a.y + (size_t)m0 * a.n + n0, (uint32_t)kLM * (uint32_t)a.n * 4u);
    const uint32_t vb = (((uint32_t)wave * 64 + 4 * (lane >> 4)) * (uint32_t)a.n + (lane & 15)) * 4u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t so = (uint32_t)(16 * i + r) * (uint32_t)a.n * 4u;
#pragma unroll
        for (int jn = 0; jn < 8; ++jn) buf_store_f32(acc[i][jn][r], by, vb + 64u * jn, so);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 8; ++jn) {
      const int col = n0 + 16 * jn + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wave * 64 + 16 * i + 4 * (lane >> 4) + r;
        if (row < a.m && col < a.n) a.y[(size_t)row * a.n + col] = acc[i][jn][r];
      }
    }
}

// ---------------------------------------------------------------------------
// large M, wide N (N >= 8192), K % 256 == 0
// ---------------------------------------------------------------------------
constexpr int kWN = 256;  // W rows per tile of the wide kernel

// MFMA with the accumulator tied to its registers (the compiler then keeps
// every accumulator in place across the unrolled K loop instead of moving it
// between register sets).  Accumulators are reused 64 MFMAs later at the
// soonest; mfma_drain() separates the last MFMAs from the epilogue reads.
__device__ __forceinline__ void mfma_tied(f32x4 &acc, const bf16x8_t &a, const bf16x8_t &b) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
#else
  (void)acc, (void)a, (void)b;
#endif
}
__device__ __forceinline__ void mfma_tied(f32x4 &acc, const f16x8_t &a, const f16x8_t &b) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
#else
  (void)acc, (void)a, (void)b;
#endif
}

// Tile 256 (tokens) x 256 (W rows), K step 32, 4 waves stacked along the
// tokens, each owning 64 x 256 as 4 x 16 blocks of v_mfma_f32_16x16x32_bf16:
// twice the W rows of k_gemm_tile per x fragment, so half the x traffic per
// MFMA.  Thread t decodes W row t (all four groups of a K step) into an LDS
// tile of 64-byte rows whose four 16-byte chunks are XOR-swizzled by row
// (conflict-free fragment reads without padding: two tiles and the
// codebooks fill the 160 KiB).  Pipeline: iteration k reads the B fragments
// of tile k & 1 in two halves, issues the gathers of step k+1, interleaves
// the 64 MFMAs of step k with the decode of step k+1 into the other tile,
// loads step k+4, one barrier.
template <class LD, bool RS, bool F16 = false>
__global__ __launch_bounds__(256) void k_gemm_wide(GemmArgs a) {
  constexpr int S = LD::S;
  using frag_t = typename std::conditional<F16, f16x8_t, bf16x8_t>::type;
  __shared__ uint4 s_cb[LD::kRows];
  __shared__ __attribute__((aligned(16))) uint4 s_w[2][kWN * 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int L = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  if (L >= a.tiles_m * a.tiles_n) return;  // whole workgroup, before any barrier
  const int m0 = (L / a.tiles_n) * kLM;
  const int n0 = (L % a.tiles_n) * kWN;
  if constexpr (LD::kUniform) {
    constexpr int BITS = LD::bits(0);
    constexpr int CBN = S << BITS;
#pragma unroll 4
    for (int r = 0; r < CBN / 256; ++r) {
      const int blk = (r * 4 + wave) * 64;
      lds_direct_16(reinterpret_cast<const uint4 *>(a.cb[blk >> BITS]) + (blk & ((1 << BITS) - 1)) + lane,
                    s_cb + blk);
    }
  } else {
    stage_ladder_lds<LD, 4>(a.cb, s_cb, wave, lane);
  }
  // W row of this thread (rows past n decode the last row: they only feed
  // output columns past n, which are never stored)
  const int wrow_c = min(n0 + tid, a.n - 1);
  const uint32_t ng = (uint32_t)a.n * a.G;
  buf_t blo[S], bhi[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    blo[t] = make_buf(LD::lo(t) ? a.lo[t] : a.hi[t], ng);
    bhi[t] = make_buf(LD::hi(t) ? a.hi[t] : a.lo[t], LD::hi(t) ? (ng + 1) / 2 : ng);
  }
  const buf_t bsc = make_buf(a.sc, 2u * a.n * a.nblk);
  const buf_t bx = F16 ? make_buf(a.xh, 2u * (uint32_t)a.m_pad * (uint32_t)a.k) : make_buf(a.x, 2u * a.m * a.k);
  const uint32_t vlo = (uint32_t)wrow_c * a.G;
  const uint32_t vhi = vlo >> 1;
  const uint32_t vsc = 2u * wrow_c * a.nblk;
  // (fp16 path: the lane's 16 bytes of its token block's 1 KiB fragment
  // per K step; blocks past m_pad load the last one)
  uint32_t va[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (F16) {
      const uint32_t tb = (uint32_t)min(m0 + wave * 64 + 16 * i, a.m_pad - 16) / 16u;
      va[i] = 16u * (tb * (uint32_t)(a.k / 32) * 64u + (uint32_t)lane);
    } else {
      const int r = min(m0 + wave * 64 + 16 * i + (lane & 15), a.m - 1);
      va[i] = 2u * ((uint32_t)r * a.k + 8 * (lane >> 4));
    }
  }
  // swizzled chunk position of chunk c of tile row r
  auto wpos = [](int r, int c) { return 4 * r + (c ^ ((r >> 2) & 3)); };

  f32x4 acc[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = a.G / 4;
  const int nq = a.G / 16;
  auto load_quad = [&](int j, Quad<S> &Q) {
    j = min(j, nq - 1);
#pragma unroll
    for (int t = 0; t < S; ++t) {
      if (LD::lo(t)) Q.lo[t] = buf_u128(blo[t], vlo, 16u * j);
      if (LD::hi(t)) Q.hi[t] = buf_u64(bhi[t], vhi, 8u * j);
    }
  };
  auto load_x = [&](int ks, XStep &X) {
    ks = min(ks, nks - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) X.av[i] = buf_u128(bx, va[i], (F16 ? 1024u : 64u) * ks);
    const uint32_t blk = (uint32_t)(((uint64_t)ks * a.smagic) >> 32);
    X.sc = buf_u16(bsc, vsc, 2u * blk);
  };
  // group g of the thread's row in step s of quad Q (one codebook vector per
  // stage)
  auto gather1 = [&](const Quad<S> &Q, int s, int g, uint4 (&vg)[S]) {
#pragma unroll
    for (int t = 0; t < S; ++t) {
      uint32_t idx = 0;
      if (LD::lo(t)) {
        const uint32_t lw = s == 0 ? Q.lo[t].x : s == 1 ? Q.lo[t].y : s == 2 ? Q.lo[t].z : Q.lo[t].w;
        idx = (lw >> (8 * g)) & 0xffu;
      }
      if (LD::hi(t)) {
        const uint32_t hw = s < 2 ? Q.hi[t].x : Q.hi[t].y;
        idx |= ((hw >> (4 * (4 * (s & 1) + g))) & 0xfu) << LD::hshift(t);
      }
      vg[t] = s_cb[LD::off(t) + idx];
    }
  };
  // the four groups of the thread's row in step s of quad Q
  auto gather = [&](const Quad<S> &Q, int s, uint4 (&v)[4][S]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) gather1(Q, s, g, v[g]);
  };
  auto decode = [&](int g, const uint4 (&v)[S], uint32_t sc, uint4 *wt) {
    if constexpr (F16) wt[wpos(tid, g)] = RS ? group_to_f16_scaled<S>(v, h2f(sc), a.rs) : group_to_f16<S>(v, sc);
    else wt[wpos(tid, g)] = RS ? group_to_bf16_scaled<S>(v, h2f(sc), a.rs) : group_to_bf16<S>(v, h2f(sc));
  };
  auto read_b2 = [&](const uint4 *wr, int half, int j0, frag_t (&bfr)[8]) {
#pragma unroll
    for (int j = j0; j < j0 + 2; ++j)
      bfr[j] = __builtin_bit_cast(frag_t, wr[wpos(16 * (8 * half + j) + (lane & 15), lane >> 4)]);
  };
  auto read_b = [&](const uint4 *wr, int half, frag_t (&bfr)[8]) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) read_b2(wr, half, j, bfr);
  };
  auto mma = [&](const XStep &X, const frag_t (&bfr)[8], int half, int i) {
    const frag_t afr = __builtin_bit_cast(frag_t, X.av[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) mfma_tied(acc[i][8 * half + j], afr, bfr[j]);
  };
  // Iteration ks, two phases around one barrier.  A: the reads of the second
  // half of step ks (tile ks & 1) into BB are issued, then the MFMAs of the
  // first half (fragments in BA) alternate with the decode of step ks+1
  // (codebook vectors gathered one iteration earlier, in v) into tile
  // (ks+1) & 1; the global loads of step ks+4 (and of a quad of index steps)
  // go out after the first MFMA group (x of step ks+3 into the registers
  // step ks-1 used; an index quad into the quad register set whose last
  // step was gathered in the previous iteration).  Barrier: tile ks+1 is complete, and
  // every read of tile ks & 1 has finished (it is rewritten in iteration
  // ks+1).  B: four rounds of four LDS reads (two B fragments of the first
  // half of step ks+1 into BA, the gathers of one group of step ks+2 into v)
  // each followed by eight MFMAs of the second half (BB), so a wave never has
  // more LDS reads in flight than the 15 the counter tracks and the MFMAs
  // start at once.
  auto iter = [&](int ks, const XStep &Xm, const XStep &Xd, XStep &Xl, const Quad<S> &Qg, int sg, Quad<S> &Qn,
                  bool quad_load, frag_t (&BA)[8], frag_t (&BB)[8], uint4 (&v)[4][S]) {
    const uint4 *wr = s_w[ks & 1];
    uint4 *ww = s_w[(ks + 1) & 1];
    read_b(wr, 1, BB);
    sched_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mma(Xm, BA, 0, i);
      sched_fence();
      decode(i, v[i], Xd.sc, ww);
      sched_fence();
      if (i == 0) {
        // x first: loads complete in issue order, so the next x load waited
        // on after an index quad (from HBM) is then issued an iteration
        // later and the quad gets four iterations instead of three
        load_x(ks + 3, Xl);
        if (quad_load) load_quad((ks + 6) / 4, Qn);
        sched_fence();
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      read_b2(ww, 0, 2 * i, BA);
      gather1(Qg, sg, i, v[i]);
      sched_fence();
      mma(Xm, BB, 1, i);
      sched_fence();
    }
  };

  Quad<S> Q0, Q1;
  XStep X0, X1, X2, X3;
  load_quad(0, Q0);
  load_quad(1, Q1);
  load_x(0, X0);
  load_x(1, X1);
  load_x(2, X2);
  wait_all_memory();  // codebook (LDS-direct) has landed (and the first steps)
  __syncthreads();
  uint4 v[4][S];
  gather(Q0, 0, v);
#pragma unroll
  for (int g = 0; g < 4; ++g) decode(g, v[g], X0.sc, s_w[0]);
  gather(Q0, 1, v);
  __syncthreads();
  frag_t BA[8], BB[8];
  read_b(s_w[0], 0, BA);
  // eight steps (two quads) per trip: iteration ks gathers step ks+2, so quad
  // Q0 (steps ks..ks+3) is last gathered in iteration ks+1 and refilled in
  // iteration ks+2 with steps ks+8..ks+11 (first gathered in iteration
  // ks+6); Q1 likewise in iterations ks+5 / ks+6 / ks+10
  for (int ks = 0; ks < nks; ks += 8) {
    iter(ks + 0, X0, X1, X3, Q0, 2, Q0, false, BA, BB, v);
    iter(ks + 1, X1, X2, X0, Q0, 3, Q0, false, BA, BB, v);
    iter(ks + 2, X2, X3, X1, Q1, 0, Q0, true, BA, BB, v);   // quad (ks+8)/4 -> Q0
    iter(ks + 3, X3, X0, X2, Q1, 1, Q1, false, BA, BB, v);
    iter(ks + 4, X0, X1, X3, Q1, 2, Q1, false, BA, BB, v);
    iter(ks + 5, X1, X2, X0, Q1, 3, Q1, false, BA, BB, v);
    iter(ks + 6, X2, X3, X1, Q0, 0, Q1, true, BA, BB, v);   // quad (ks+12)/4 -> Q1
    iter(ks + 7, X3, X0, X2, Q0, 1, Q1, false, BA, BB, v);
    // The hardware does not interlock a read of an accumulator after the
    // MFMA that writes it, and the compiler cannot see into the MFMA asm: at
    // the loop exit it may copy accumulators (register-allocation moves)
    // right after the last MFMAs.  32 wait cycles at the end of every trip
    // (inside the loop, so before any such copy) cover the MFMA latency.
    sched_fence();
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
#endif
    sched_fence();
  }
  // the same wait before the epilogue reads, tied to every block of eight
  // accumulators
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                   "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[i][8]), "+a"(acc[i][9]), "+a"(acc[i][10]), "+a"(acc[i][11]), "+a"(acc[i][12]),
                   "+a"(acc[i][13]), "+a"(acc[i][14]), "+a"(acc[i][15]));
  }
#endif
  if constexpr (F16) token_factors(a, m0, wave, lane, acc);
  // Tiles lying wholly inside y (every row < m, every column < n) store
  // through a descriptor based at the tile's first element without per-store
  // tests: the lane's offset is fixed, rows step by a scalar offset, columns
  // by an immediate.  Edge tiles take the tested stores below.
  if (m0 + kLM <= a.m && n0 + kWN <= a.n && (uint64_t)kLM * a.n * 4 < (1u << 31)) {
    const buf_t by = make_buf(a.y + (size_t)m0 * a.n + n0, (uint32_t)kLM * (uint32_t)a.n * 4u);
    const uint32_t vb = (((uint32_t)wave * 64 + 4 * (lane >> 4)) * (uint32_t)a.n + (lane & 15)) * 4u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t so = (uint32_t)(16 * i + r) * (uint32_t)a.n * 4u;
#pragma unroll
        for (int jn = 0; jn < 16; ++jn) buf_store_f32(acc[i][jn][r], by, vb + 64u * jn, so);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 16; ++jn) {
      const int col = n0 + 16 * jn + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wave * 64 + 16 * i + 4 * (lane >> 4) + r;
        if (row < a.m && col < a.n) a.y[(size_t)row * a.n + col] = acc[i][jn][r];
      }
    }
}

// ---------------------------------------------------------------------------
// small M
// ---------------------------------------------------------------------------
constexpr int kSWaves = 8;

// Registers of one 128-column super step for one lane: index bits of its 4
// consecutive groups per stage, their scale, and 32 x values of its token.
template <int S>
struct SmallRegs {
  uint32_t lo[S];  // 4 low bytes (8/12-bit) or, 16-bit, 2 indices in lo and 2 in hi
  uint32_t hi[S];  // 12-bit: 4 nibbles; 16-bit: indices 2 and 3
  uint32_t sc;     // fp16 bits (all 4 groups share a block: scale_block % 32 == 0)
  uint4 av[4];     // x[token][128 J + 32 q .. + 32)
};

template <int S, int BITS>
__device__ __forceinline__ void small_load(const GemmArgs &a, int J, int q, int wrow_c, int tok_c, SmallRegs<S> &R) {
  const int g = 16 * J + 4 * q;
  const size_t f = (size_t)wrow_c * a.G + g;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    if (BITS == 16) {
      const uint2 v = *reinterpret_cast<const uint2 *>(a.i16[t] + f);
      R.lo[t] = v.x;
      R.hi[t] = v.y;
    } else {
      R.lo[t] = *reinterpret_cast<const uint32_t *>(a.lo[t] + f);
      R.hi[t] = (BITS == 12) ? (uint32_t) * reinterpret_cast<const uint16_t *>(a.hi[t] + (f >> 1)) : 0u;
    }
  }
  R.sc = a.sc[(size_t)wrow_c * a.nblk + scale_blk(a, g)];
  const uint4 *px = reinterpret_cast<const uint4 *>(a.x + (size_t)tok_c * a.k + 8 * g);
#pragma unroll
  for (int v = 0; v < 4; ++v) R.av[v] = px[v];
}

// 1 <= m <= 16.  Persistent workgroups of 8 waves walk 16-row slabs of W.
// A 128-column super step J holds 16 groups; lane l (W row and token l%16,
// slot q = l/16) takes groups 16J + 4q + r and feeds group r to the r-th
// v_mfma_f32_16x16x32_bf16 of the step in k-slot q (the same permutation of
// k for A and B, so the contraction is unchanged).  Wave w takes super
// steps w, w+8, ...; the next one loads while the current one decodes
// (LDS codebook gathers straight into B fragments) and multiplies.  The
// eight wave partials are added in LDS in a fixed order.
// Requires K % 128 == 0 and scale_block % 32 == 0 (else k_gemm_small_gen).
template <int S, int BITS, bool CB_LDS>
__global__ __launch_bounds__(kSWaves * 64) void k_gemm_small(GemmArgs a) {
  __shared__ uint4 s_cb[CB_LDS ? (S << BITS) : 1];
  __shared__ float s_red[kSWaves][16][17];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  if (CB_LDS) {
    constexpr int CBN = S << BITS;
#pragma unroll 4
    for (int r = 0; r < (CBN + kSWaves * 64 - 1) / (kSWaves * 64); ++r) {
      const int blk = (r * kSWaves + wave) * 64;
      if (blk < CBN)
        lds_direct_16(reinterpret_cast<const uint4 *>(a.cb[blk >> BITS]) + (blk & ((1 << BITS) - 1)) + lane,
                      s_cb + blk);
    }
    wait_all_memory();
    __syncthreads();
  }
  const int j16 = lane & 15;  // W row within the slab = token of the A fragment
  const int q = lane >> 4;
  const int tok_c = j16 < a.m ? j16 : a.m - 1;  // tokens past m only feed unstored outputs
  const int nJ = a.G / 16;
  const int nslabs = (a.n + 15) / 16;

  // the group's weights as bf16 hi + lo parts (split_bf16)
  auto decode = [&](const SmallRegs<S> &R, int r, uint4 &hi, uint4 &lo) {
    float w[8];
#pragma unroll
    for (int t = 0; t < S; ++t) {
      uint32_t idx;
      if (BITS == 16) idx = (r < 2 ? (R.lo[t] >> (16 * r)) : (R.hi[t] >> (16 * (r - 2)))) & 0xffffu;
      else {
        idx = (R.lo[t] >> (8 * r)) & 0xffu;
        if (BITS == 12) idx |= ((R.hi[t] >> (4 * r)) & 0xfu) << 8;
      }
      const uint4 v = CB_LDS ? s_cb[(BITS ? (t << BITS) : a.cboff[t]) + idx] : reinterpret_cast<const uint4 *>(a.cb[t])[idx];
      const uint32_t hv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c0 = h2f(hv[e] & 0xffffu), c1 = h2f(hv[e] >> 16);
        w[2 * e] = (t == 0) ? c0 : w[2 * e] + c0;
        w[2 * e + 1] = (t == 0) ? c1 : w[2 * e + 1] + c1;
      }
    }
    const float sf = h2f(R.sc);
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] *= sf;
    split_bf16(w, hi, lo);
  };

  for (int slab = blockIdx.x; slab < nslabs; slab += gridDim.x) {
    const int n0 = slab * 16;
    const int wrow = n0 + j16;
    const int wrow_c = wrow < a.n ? wrow : a.n - 1;  // rows past n only feed unstored outputs
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // this wave's super steps: J_i = wave + 8 i; ring of four register sets,
    // three super steps in flight while one is decoded and multiplied
    const int nmine = wave < nJ ? (nJ - 1 - wave) / kSWaves + 1 : 0;
    SmallRegs<S> R0, R1, R2, R3;
    // unconditional prefetch (past this wave's last super step it reloads
    // the last one), so no branch surrounds the loads
    auto load = [&](int i, SmallRegs<S> &R) {
      small_load<S, BITS>(a, wave + kSWaves * (i < nmine ? i : nmine - 1), q, wrow_c, tok_c, R);
      sched_fence();  // keep the prefetch here, three super steps ahead of its use
    };
    auto run = [&](const SmallRegs<S> &R) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint4 hi, lo;
        decode(R, r, hi, lo);
        const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, R.av[r]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8_t, hi), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8_t, lo), acc, 0, 0, 0);
      }
    };
    if (nmine > 0) {  // wave-uniform; every wave still reaches both barriers below
      load(0, R0);
      load(1, R1);
      load(2, R2);
      int i = 0;
      for (; i + 4 <= nmine; i += 4) {  // single exit (see the large-M kernel)
        load(i + 3, R3);
        run(R0);
        load(i + 4, R0);
        run(R1);
        load(i + 5, R1);
        run(R2);
        load(i + 6, R2);
        run(R3);
      }
      const int rem = nmine - i;  // sets R0, R1, R2 hold super steps i, i+1, i+2
      if (rem > 0) run(R0);
      if (rem > 1) run(R1);
      if (rem > 2) run(R2);
    }
    // lane holds D[token 4*(lane/16)+r][W row lane%16]
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[wave][4 * (lane >> 4) + r][lane & 15] = acc[r];
    __syncthreads();
    if (tid < 256) {
      const int ti = tid >> 4, wj = tid & 15;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) sum += s_red[w][ti][wj];
      if (ti < a.m && n0 + wj < a.n) a.y[(size_t)ti * a.n + n0 + wj] = sum;
    }
    __syncthreads();
  }
}

// 1 <= m <= 64 tokens, K % 256 == 0, scale_block % 128 == 0, LDS codebooks
// of 8/12-bit indices.  A unit is 16 W rows over a K range; lane l decodes,
// per 32-column K step, group l / 16 of row l % 16 straight into a B fragment
// of v_mfma_f32_16x16x32_bf16 (no LDS round trip) and multiplies it with the
// A fragments of TB blocks of 16 tokens (lane l loads 8 x values of token
// l % 16 of each block).  A workgroup's eight waves take its units times KP K
// parts; the KP partial tiles of a unit are added in LDS in a fixed order at
// the end.
// Index bytes: the four lanes of a row need the same 16 bytes per four
// steps, so instead of four identical loads each wave stages its rows' bytes
// for eight steps (two quads of low bytes, one 16-byte run of high nibbles
// per stage) into a two-slot LDS ring with LDS-direct loads, one unique
// 16-byte piece per lane, a trip ahead, and reads them back (a broadcast LDS
// read per row).  x is loaded three steps ahead; the scale (one per 128
// columns at most) once per quad, a trip ahead.
template <int S>
struct FewQuad {
  uint4 lo[S];
  uint2 hi[S];
  uint32_t sc;  // fp16 scale of the lane's row
};
template <int TB>
struct FewStep {
  uint4 av[TB];  // A fragments of the token blocks
};

template <class LD, bool RS, int TB>
__global__ __launch_bounds__(kSWaves * 64) void k_gemm_few(GemmArgs a, int units_per_wg, int kp) {
  constexpr int S = LD::S;
  // index planes staged per stage: two quads of low bytes (stages with a
  // byte plane) and one 16-byte run of nibbles (stages with a nibble plane)
  constexpr bool kAnyLo = LD::lo(0) || LD::lo(1) || LD::lo(2) || LD::lo(3);
  constexpr int HI = (LD::hi(0) || LD::hi(1) || LD::hi(2) || LD::hi(3)) ? 1 : 0;
  constexpr int SLOT = (2 + HI) * S * 16;  // uint4 per wave and slot: 2 lo quads (+ hi pair) x S stages x 16 rows
  constexpr int RED = (kSWaves * 16 * 17 * 4 + 15) / 16;  // uint4 of the final reduction (aliases the ring)
  constexpr int STAGE = kSWaves * 2 * SLOT > RED ? kSWaves * 2 * SLOT : RED;
  __shared__ uint4 s_cb[LD::kRows];
  __shared__ uint4 s_stage[STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  if constexpr (LD::kUniform) {
    constexpr int BITS = LD::bits(0);
    constexpr int CBN = S << BITS;
#pragma unroll 4
    for (int r = 0; r < (CBN + kSWaves * 64 - 1) / (kSWaves * 64); ++r) {
      const int blk = (r * kSWaves + wave) * 64;
      if (blk < CBN)
        lds_direct_16(reinterpret_cast<const uint4 *>(a.cb[blk >> BITS]) + (blk & ((1 << BITS) - 1)) + lane,
                      s_cb + blk);
    }
  } else {
    stage_ladder_lds<LD, kSWaves>(a.cb, s_cb, wave, lane);
  }
  const int units = (a.n + 15) / 16;
  const int nks = a.G / 4;
  const int steps = nks / kp;        // K steps per part (a multiple of 8)
  const int trips = steps / 8;
  const int ui = wave / kp;          // unit slot of this wave in the workgroup
  const int part = wave % kp;
  const int unit = blockIdx.x * units_per_wg + ui;
  const bool active = ui < units_per_wg && unit < units;  // wave-uniform
  const int r16 = lane & 15;
  const int q = lane >> 4;           // k chunk of the lane within a K step
  const int ks0 = part * steps;
  const int row = min((active ? unit : 0) * 16 + r16, a.n - 1);

  const buf_t bsc = make_buf(a.sc, 2u * a.n * a.nblk);
  const buf_t bx = make_buf(a.x, 2u * a.m * a.k);
  const uint32_t vsc = 2u * row * a.nblk;
  uint32_t vx[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int tok = min(16 * tb + r16, a.m - 1);  // tokens past m only feed unstored outputs
    vx[tb] = 2u * ((uint32_t)tok * a.k + 8 * q);
  }
  // staging source of this lane: row r16, stage q (lanes q < S take part)
  const int sq = q < S ? q : 0;
  const uint8_t *src_lo = a.lo[0], *src_hi = HI ? a.hi[0] : a.lo[0];
  bool lane_lo = LD::lo(0), lane_hi = LD::hi(0);  // planes of this lane's stage
#pragma unroll
  for (int t = 1; t < S; ++t)
    if (sq == t) {
      src_lo = a.lo[t];
      if (HI) src_hi = a.hi[t];
      lane_lo = LD::lo(t);
      lane_hi = LD::hi(t);
    }
  src_lo += (size_t)row * a.G;
  if (HI) src_hi += ((size_t)row * a.G) >> 1;

  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // stage the index bytes of trip i (quads 2i, 2i+1 of this part, clamped)
  // into slot i & 1 of this wave's ring
  auto stage = [&](int i) {
    uint4 *base = s_stage + (wave * 2 + (i & 1)) * SLOT;
    const int j0 = ks0 / 4 + min(2 * i, steps / 4 - 2);  // first quad (trips hold two)
    // (a plane instruction is issued whenever some stage has that plane, so
    // the count of loads per trip is fixed; lanes of stages without it are
    // masked off)
    if (q < S) {
      if (kAnyLo) {
        if (LD::kUniform || lane_lo) {
          lds_direct_16(src_lo + 16 * j0, base);
          lds_direct_16(src_lo + 16 * (j0 + 1), base + S * 16);
        }
      }
      if (HI) {
        if (LD::kUniform || lane_hi) lds_direct_16(src_hi + 8 * j0, base + 2 * S * 16);
      }
    }
  };
  constexpr int kStageLoads = (kAnyLo ? 2 : 0) + HI;
  auto load_sc = [&](int i, uint32_t (&sc)[2]) {
    const int j0 = ks0 / 4 + min(2 * i, steps / 4 - 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t blk = (uint32_t)(((uint64_t)(4 * (j0 + h)) * a.smagic) >> 32);  // (128 j) / scale_block
      sc[h] = buf_u16(bsc, vsc, 2u * blk);
    }
  };
  // the staged bytes of trip i: this lane's row, every stage
  auto read_trip = [&](int i, FewQuad<S> &Q0, FewQuad<S> &Q1) {
    const uint4 *base = s_stage + (wave * 2 + (i & 1)) * SLOT;
#pragma unroll
    for (int t = 0; t < S; ++t) {
      if (LD::lo(t)) {
        Q0.lo[t] = base[t * 16 + r16];
        Q1.lo[t] = base[S * 16 + t * 16 + r16];
      }
      if (LD::hi(t)) {
        const uint4 h = base[2 * S * 16 + t * 16 + r16];
        Q0.hi[t] = make_uint2(h.x, h.y);
        Q1.hi[t] = make_uint2(h.z, h.w);
      }
    }
  };
  // With two or more token blocks, x of a pair of K steps (2u, 2u + 1) is
  // loaded with the odd token rows taking the other step first, so that each
  // load reads both halves of the 128-byte lines of its sixteen rows (every
  // row reading the same half costs the stream up to 30 %); swap_pair puts
  // the steps back in place before their use.  One block (16 tokens or
  // fewer) keeps the plain order: it gained nothing at 16 tokens, and with
  // fewer the rows past the last token (which repeat it) would touch both
  // halves of its lines.
  constexpr bool kPair = TB >= 2;
  const bool odd_row = (r16 & 1) != 0;
  auto load_step = [&](int i, FewStep<TB> &X) {
    const int ks = ks0 + min(i, steps - 1);  // ks0 is even
    const uint32_t sel = kPair ? (uint32_t)(ks & 1) ^ (uint32_t)odd_row : 0u;
    const uint32_t kb = kPair ? (uint32_t)(ks & ~1) : (uint32_t)ks;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) X.av[tb] = buf_u128(bx, vx[tb] + 64u * sel, 64u * kb);
  };
  auto swap_pair = [&](FewStep<TB> &A, FewStep<TB> &B) {
    if constexpr (!kPair) return;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const uint4 u = A.av[tb], v = B.av[tb];
      A.av[tb] = odd_row ? v : u;
      B.av[tb] = odd_row ? u : v;
    }
  };
  // decode the lane's group in step s (0..3) of quad Q and multiply with
  // every token block
  auto step = [&](const FewQuad<S> &Q, int s, const FewStep<TB> &X) {
    uint4 v[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
      uint32_t idx = 0;
      if (LD::lo(t)) {
        const uint4 lw4 = Q.lo[t];
        const uint32_t lw = s == 0 ? lw4.x : s == 1 ? lw4.y : s == 2 ? lw4.z : lw4.w;
        idx = (lw >> (8 * q)) & 0xffu;
      }
      if (LD::hi(t)) {
        const uint32_t hw = s < 2 ? Q.hi[t].x : Q.hi[t].y;
        idx |= ((hw >> (4 * (4 * (s & 1) + q))) & 0xfu) << LD::hshift(t);
      }
      v[t] = s_cb[LD::off(t) + idx];
    }
    const float sf = h2f(Q.sc);
    // the weights as bf16 hi + lo, two MFMAs per token block
    float w[8];
    if constexpr (RS) group_to_f32_scaled<S>(v, sf, a.rs, w);
    else group_to_f32<S>(v, sf, w);
    uint4 hi, lo;
    split_bf16(w, hi, lo);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, X.av[tb]);
      acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8_t, hi), acc[tb], 0, 0, 0);
      acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8_t, lo), acc[tb], 0, 0, 0);
    }
  };

  FewQuad<S> Q0, Q1;
  FewStep<TB> X0, X1, X2, X3;
  uint32_t nsc[2];
  if (active) {
    stage(0);
    load_sc(0, nsc);
    load_step(0, X0);
    load_step(1, X1);
    load_step(2, X2);
  }
  wait_all_memory();  // codebook (LDS-direct) and trip 0 have landed
  __syncthreads();
  if (active) {  // wave-uniform
    // one trip (two quads, eight steps) per iteration: trip i+1 is staged
    // and its scales loaded first.  Loads complete in issue order, and the
    // loads issued after trip i's staging are trip i's two scale loads, the
    // 8 TB x loads of iteration i-1 and the staging and scales of trip i+1:
    // waiting until at most that many are outstanding means trip i landed
    for (int i = 0; i < trips; ++i) {
      Q0.sc = nsc[0];
      Q1.sc = nsc[1];
      if (i + 1 < trips) {
        stage(i + 1);
        load_sc(i + 1, nsc);
      }
      sched_fence();
      // (the last trip stages nothing more, so fewer loads follow its own)
      constexpr int kAfter = 2 + 8 * TB + kStageLoads + 2;
      constexpr int kAfterLast = 2 + 8 * TB;
      if (i + 1 < trips) {
        if (i > 0) wait_vmem<(kAfter < 63 ? kAfter : 63)>();
      } else if (i > 0) {
        wait_vmem<(kAfterLast < 63 ? kAfterLast : 63)>();
      }
      read_trip(i, Q0, Q1);
      sched_fence();
      const int k = 8 * i;
      load_step(k + 3, X3);
      swap_pair(X0, X1);
      step(Q0, 0, X0);
      load_step(k + 4, X0);
      step(Q0, 1, X1);
      load_step(k + 5, X1);
      swap_pair(X2, X3);
      step(Q0, 2, X2);
      load_step(k + 6, X2);
      step(Q0, 3, X3);
      load_step(k + 7, X3);
      swap_pair(X0, X1);
      step(Q1, 0, X0);
      load_step(k + 8, X0);
      step(Q1, 1, X1);
      load_step(k + 9, X1);
      swap_pair(X2, X3);
      step(Q1, 2, X2);
      load_step(k + 10, X2);
      step(Q1, 3, X3);
    }
  }
  // every staged load has landed and every wave has left its ring before the
  // ring holds the reduction
  wait_all_memory();
  __syncthreads();
  float (*s_red)[16][17] = reinterpret_cast<float (*)[16][17]>(s_stage);
  // per token block: lane holds D[token 4 (lane / 16) + r][row lane % 16];
  // part 0 of each unit adds the KP parts in order
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[wave][4 * (lane >> 4) + r][lane & 15] = acc[tb][r];
    __syncthreads();
    if (active && part == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ti = 16 * tb + 4 * (lane >> 4) + r;
        float sum = 0.f;
        for (int h = 0; h < kp; ++h) sum += s_red[wave + h][4 * (lane >> 4) + r][lane & 15];
        const int col = unit * 16 + (lane & 15);
        if (ti < a.m && col < a.n) a.y[(size_t)ti * a.n + col] = sum;
      }
    }
    __syncthreads();
  }
}

// General small-M path (any K % 8 == 0, any scale block): one group per lane
// per 32-column K step, byte-wise index loads.  BITS = 0: residual ladders
// of per-stage widths and stage scales.
template <int S, int BITS, bool CB_LDS>
__global__ __launch_bounds__(kSWaves * 64) void k_gemm_small_gen(GemmArgs a) {
  __shared__ uint4 s_cb[CB_LDS ? (BITS ? (S << BITS) : kLadderCbRows) : 1];
  __shared__ float s_red[kSWaves][16][17];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  if (CB_LDS) {
    if constexpr (BITS != 0) {
      for (int i = tid; i < (S << BITS); i += kSWaves * 64)
        s_cb[i] = reinterpret_cast<const uint4 *>(a.cb[i >> BITS])[i & ((1 << BITS) - 1)];
    } else {
      stage_ladder_codebooks(a, s_cb, tid, kSWaves * 64);
    }
    __syncthreads();
  }
  const int nks = (a.G + 3) / 4;
  const int tok = lane & 15;
  const int q = lane >> 4;
  const int nslabs = (a.n + 15) / 16;
  for (int slab = blockIdx.x; slab < nslabs; slab += gridDim.x) {
    const int n0 = slab * 16;
    const int wrow = n0 + tok;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = wave; ks < nks; ks += kSWaves) {
      const int g = ks * 4 + q;
      uint4 av = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0), lo = make_uint4(0, 0, 0, 0);
      if (g < a.G) {
        if (tok < a.m) av = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok * a.k + 8 * g);
        if (wrow < a.n) {
          float w[8];
          decode_group_f32<S, BITS, CB_LDS>(a, s_cb, wrow, g, w);
          split_bf16(w, hi, lo);
        }
      }
      const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, av);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8_t, hi), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8_t, lo), acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[wave][4 * (lane >> 4) + r][lane & 15] = acc[r];
    __syncthreads();
    if (tid < 256) {
      const int ti = tid >> 4, wj = tid & 15;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) sum += s_red[w][ti][wj];
      if (ti < a.m && n0 + wj < a.n) a.y[(size_t)ti * a.n + n0 + wj] = sum;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
static GemmArgs make_gemm_args(const WView &w, const uint16_t *x, int m, float *y) {
  GemmArgs a{};
  for (int t = 0; t < VQ_MAX_STAGES; ++t) {
    a.lo[t] = w.lo[t];
    a.hi[t] = w.hi[t];
    a.i16[t] = w.i16[t];
    a.cb[t] = w.cb[t];
  }
  a.sc = w.sc;
  a.x = x;
  a.y = y;
  a.m = m;
  a.n = w.n;
  a.k = w.k;
  a.G = w.G;
  a.S = w.S;
  a.nblk = w.nblk;
  a.bs = w.bs;
  const int gb = w.bs / 8;
  a.gshift = (gb & (gb - 1)) == 0 ? __builtin_ctz((unsigned)gb) : -1;
  const uint64_t spb = w.bs % 32 == 0 ? (uint64_t)(w.bs / 32) : 1;
  a.smagic = ((uint64_t(1) << 32) + spb - 1) / spb;
  a.cbrows = 0;
  for (int t = 0; t < VQ_MAX_STAGES; ++t) {
    a.sb[t] = t < w.S ? w.sb[t] : 0;
    a.rs[t] = w.rs[t];
    a.cboff[t] = a.cbrows;
    if (t < w.S) a.cbrows += 1 << w.sb[t];
  }
  return a;
}

// The few-token unit kernel with TB token blocks; false with 16 tokens or
// fewer when the shape leaves it fewer units than half the CUs (the slab
// kernels, whose weights also enter as bf16 hi + lo parts, spread such
// shapes better).  With 17..64 tokens it takes every row count up to eight
// units per CU: the tile kernels it would leave them to round the weights
// to bf16 alone.
template <class LD, bool RS>
static bool launch_few(const GemmArgs &a, hipStream_t s) {
  const int cus = device_cu_count();
  const int units = (a.n + 15) / 16;
  if (a.m <= 16 && 2 * units < cus) return false;
  const int grid = units < cus ? units : cus;
  const int upw = (units + grid - 1) / grid;
  const int nks = a.k / 32;
  // K parts per unit: as many as the eight waves allow, each a whole number
  // of eight-step trips
  int kp = 1;
  while (kp * 2 * upw <= kSWaves && nks % (kp * 2 * 8) == 0) kp *= 2;
  if (upw * kp > kSWaves) return false;
  switch ((a.m + 15) / 16) {
    case 1: hipLaunchKernelGGL((k_gemm_few<LD, RS, 1>), dim3(grid), dim3(kSWaves * 64), 0, s, a, upw, kp); break;
    case 2: hipLaunchKernelGGL((k_gemm_few<LD, RS, 2>), dim3(grid), dim3(kSWaves * 64), 0, s, a, upw, kp); break;
    case 3: hipLaunchKernelGGL((k_gemm_few<LD, RS, 3>), dim3(grid), dim3(kSWaves * 64), 0, s, a, upw, kp); break;
    default: hipLaunchKernelGGL((k_gemm_few<LD, RS, 4>), dim3(grid), dim3(kSWaves * 64), 0, s, a, upw, kp); break;
  }
  return true;
}

// The 256 x 256 (wide) or 256 x 128 (tile) kernel for many tokens when the
// shape allows it (K % 256 == 0, scale blocks of whole K steps, K < 2^20);
// false: nothing launched.  With a.xh set (one or two stages) the fp16
// variants run on x converted by k_x_f16.  `a` has tiles_m / tiles_n / per_xcd of the
// 256 x 128 tiling.
template <class LD, bool RS>
static bool launch_tiles(const GemmArgs &a, hipStream_t s) {
  const bool buf_ok = a.k % 32 == 0 && a.bs % 32 == 0 && a.k < (1 << 20);
  if (!buf_ok || a.k % 256 != 0) return false;
  if constexpr (LD::kRows * 16 + 2 * kWN * 64 <= 163840) {
    // wide N: 256 x 256 tiles once there is at least one per CU
    const int wide_tiles = a.tiles_m * ((a.n + kWN - 1) / kWN);
    if (wide_tiles >= device_cu_count()) {
      GemmArgs w = a;
      w.tiles_n = (a.n + kWN - 1) / kWN;
      w.per_xcd = (w.tiles_m * w.tiles_n + 7) / 8;
      if constexpr (LD::S <= 2) {
        if (w.xh) {
          hipLaunchKernelGGL((k_gemm_wide<LD, RS, true>), dim3(8 * w.per_xcd), dim3(256), 0, s, w);
          return true;
        }
      }
      hipLaunchKernelGGL((k_gemm_wide<LD, RS>), dim3(8 * w.per_xcd), dim3(256), 0, s, w);
      return true;
    }
  }
  if constexpr (LD::S <= 2) {
    if (a.xh) {
      hipLaunchKernelGGL((k_gemm_tile<LD, RS, true>), dim3(8 * a.per_xcd), dim3(256), 0, s, a);
      return true;
    }
  }
  hipLaunchKernelGGL((k_gemm_tile<LD, RS>), dim3(8 * a.per_xcd), dim3(256), 0, s, a);
  return true;
}

// Ladders with an LDS kernel of their own (k_gemm_ladder.hip): false when
// the ladder has none (nothing launched).
bool launch_gemm_ladder_lds(const WView &w, const GemmArgs &a, hipStream_t s);

}  // namespace vqmm
