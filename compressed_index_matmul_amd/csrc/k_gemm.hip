// Many-token product y = x dequant(W)^T on bf16 matrix cores (GLQ page,
// "Inference kernels": tensor-core path for batched inputs, decoding codebook
// vectors straight into the matrix operands; the dense W is never written to
// memory).
//
// k_gemm_large -- m > 16.  Tile 256 (tokens) x 128 (W rows), K step 32
//   (4 groups), 4 waves in a 2 x 2 grid, each owning a 128 x 64 block of
//   v_mfma_f32_32x32x16_bf16 accumulators.  Per K step every thread decodes
//   two groups (stage sum and scale in fp32, rounded to bf16) into the LDS W
//   tile, which all four waves read as B fragments; A fragments (x) are
//   loaded from global memory straight into registers.  Tiles are ordered so
//   that consecutive tiles of one token panel land on the same XCD (its L2
//   keeps the x panel).
//
// k_gemm_small -- 1 <= m <= 16 (also vq_gemv with 2..16 bf16 tokens).
//   Persistent workgroups of 8 waves walk 16-row slabs of W; wave w takes
//   every 8th K step; per K step lane l decodes group l/16 of W row l%16
//   directly into its B fragment of v_mfma_f32_16x16x32_bf16 and loads the
//   matching 8 x values of token l%16 as its A fragment.  The eight wave
//   partials are added in LDS in a fixed order.
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
  int tiles_m, tiles_n, per_xcd;
};

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Decode group g of W row `row` to 8 bf16 (packed in a uint4).  Stage sum and
// scale in fp32 (summation starts from stage 0).
template <int S, int BITS, bool CB_LDS>
__device__ __forceinline__ uint4 decode_group_bf16(const GemmArgs &a, const uint4 *s_cb, int row, int g) {
  const size_t f = (size_t)row * a.G + g;
  float w[8];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const uint32_t idx = load_index(BITS, a.lo[t], a.hi[t], a.i16[t], f);
    const uint4 v = CB_LDS ? s_cb[(t << BITS) + idx] : reinterpret_cast<const uint4 *>(a.cb[t])[idx];
    const uint32_t hv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c0 = h2f(hv[e] & 0xffffu), c1 = h2f(hv[e] >> 16);
      w[2 * e] = (t == 0) ? c0 : w[2 * e] + c0;
      w[2 * e + 1] = (t == 0) ? c1 : w[2 * e + 1] + c1;
    }
  }
  const float s = h2f(a.sc[(size_t)row * a.nblk + (8 * g) / a.bs]);
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = f2bf(s * w[2 * e]) | (f2bf(s * w[2 * e + 1]) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// large M
// ---------------------------------------------------------------------------
constexpr int kLM = 256, kLN = 128;
constexpr int kWP = 40;  // bf16 per W-tile row in LDS: 32 + 8 pad (80 B: conflict-free b128)

template <int S, int BITS, bool CB_LDS>
__global__ __launch_bounds__(256) void k_gemm_large(GemmArgs a) {
  __shared__ uint4 s_cb[CB_LDS ? (S << BITS) : 1];
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kLN * kWP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  if (L >= a.tiles_m * a.tiles_n) return;  // whole workgroup, before any barrier
  const int m0 = (L / a.tiles_n) * kLM;
  const int n0 = (L % a.tiles_n) * kLN;
  const int wm = wave >> 1, wn = wave & 1;

  if (CB_LDS) {
    for (int i = tid; i < (S << BITS); i += 256)
      s_cb[i] = reinterpret_cast<const uint4 *>(a.cb[i >> BITS])[i & ((1 << BITS) - 1)];
    __syncthreads();
  }
  const int drow = tid >> 1;      // W-tile row decoded by this thread
  const int dg = 2 * (tid & 1);   // first of its two groups in the K step
  const int wrow = n0 + drow;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nks = (a.G + 3) / 4;
  for (int ks = 0; ks < nks; ++ks) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int g = ks * 4 + dg + u;
      uint4 pk = make_uint4(0, 0, 0, 0);
      if (wrow < a.n && g < a.G) pk = decode_group_bf16<S, BITS, CB_LDS>(a, s_cb, wrow, g);
      *reinterpret_cast<uint4 *>(&s_w[drow * kWP + 8 * (dg + u)]) = pk;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int col = ks * 32 + 16 * kk + 8 * (lane >> 5);
      bf16x8_t bfr[2];
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        bfr[jn] = *reinterpret_cast<const bf16x8_t *>(&s_w[(wn * 64 + 32 * jn + (lane & 31)) * kWP + 16 * kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 128 + 32 * i + (lane & 31);
        uint4 av = make_uint4(0, 0, 0, 0);
        if (row < a.m && col < a.k) av = *reinterpret_cast<const uint4 *>(a.x + (size_t)row * a.k + col);
        const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bfr[jn], acc[i][jn], 0, 0, 0);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int col = n0 + wn * 64 + 32 * jn + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < a.m && col < a.n) a.y[(size_t)row * a.n + col] = acc[i][jn][r];
      }
    }
}

// ---------------------------------------------------------------------------
// small M
// ---------------------------------------------------------------------------
constexpr int kSWaves = 8;

template <int S, int BITS, bool CB_LDS>
__global__ __launch_bounds__(kSWaves * 64) void k_gemm_small(GemmArgs a) {
  __shared__ uint4 s_cb[CB_LDS ? (S << BITS) : 1];
  __shared__ float s_red[kSWaves][16][17];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (CB_LDS) {
    for (int i = tid; i < (S << BITS); i += kSWaves * 64)
      s_cb[i] = reinterpret_cast<const uint4 *>(a.cb[i >> BITS])[i & ((1 << BITS) - 1)];
    __syncthreads();
  }
  const int nks = (a.G + 3) / 4;
  const int tok = lane & 15;   // A row (token) and B column (W row) of this lane
  const int q = lane >> 4;     // group within the K step
  const int nslabs = (a.n + 15) / 16;
  for (int slab = blockIdx.x; slab < nslabs; slab += gridDim.x) {
    const int n0 = slab * 16;
    const int wrow = n0 + tok;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = wave; ks < nks; ks += kSWaves) {
      const int g = ks * 4 + q;
      uint4 av = make_uint4(0, 0, 0, 0), bv = make_uint4(0, 0, 0, 0);
      if (g < a.G) {
        if (tok < a.m) av = *reinterpret_cast<const uint4 *>(a.x + (size_t)tok * a.k + 8 * g);
        if (wrow < a.n) bv = decode_group_bf16<S, BITS, CB_LDS>(a, s_cb, wrow, g);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                    __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
    }
    // lane holds D[token 4*(lane/16)+r][W row lane%16]
#pragma unroll
    for (int r = 0; r < 4; ++r) s_red[wave][4 * (lane >> 4) + r][lane & 15] = acc[r];
    __syncthreads();
    if (tid < 256) {
      const int ti = tid >> 4, wj = tid & 15;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) s += s_red[w][ti][wj];
      if (ti < a.m && n0 + wj < a.n) a.y[(size_t)ti * a.n + n0 + wj] = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dispatch
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
  return a;
}

template <int S, int BITS, bool CB_LDS>
static void launch_gemm_sb(const GemmArgs &a0, hipStream_t s) {
  GemmArgs a = a0;
  if (a.m <= 16) {
    const int nslabs = (a.n + 15) / 16;
    int nwg = device_cu_count();
    if (nwg > nslabs) nwg = nslabs;
    hipLaunchKernelGGL((k_gemm_small<S, BITS, CB_LDS>), dim3(nwg), dim3(kSWaves * 64), 0, s, a);
  } else {
    a.tiles_m = (a.m + kLM - 1) / kLM;
    a.tiles_n = (a.n + kLN - 1) / kLN;
    const int total = a.tiles_m * a.tiles_n;
    a.per_xcd = (total + 7) / 8;
    hipLaunchKernelGGL((k_gemm_large<S, BITS, CB_LDS>), dim3(8 * a.per_xcd), dim3(256), 0, s, a);
  }
}

// Codebooks of every stage fit in LDS next to the tiles (<= 128 KiB).
template <int S, int BITS>
constexpr bool kCbFits = BITS != 16 && (S << BITS) * 16 <= 131072;

template <int BITS>
static void launch_gemm_bits(const WView &w, const GemmArgs &a, hipStream_t s) {
  switch (w.S) {
    case 1: launch_gemm_sb<1, BITS, kCbFits<1, BITS>>(a, s); break;
    case 2: launch_gemm_sb<2, BITS, kCbFits<2, BITS>>(a, s); break;
    case 3: launch_gemm_sb<3, BITS, kCbFits<3, BITS>>(a, s); break;
    default: launch_gemm_sb<4, BITS, kCbFits<4, BITS>>(a, s); break;
  }
}

hipError_t launch_gemm(const WView &w, const uint16_t *x, int m, float *y, hipStream_t s) {
  const GemmArgs a = make_gemm_args(w, x, m, y);
  if (w.bits == 8) launch_gemm_bits<8>(w, a, s);
  else if (w.bits == 12) launch_gemm_bits<12>(w, a, s);
  else launch_gemm_bits<16>(w, a, s);
  return hipGetLastError();
}

}  // namespace vqmm
