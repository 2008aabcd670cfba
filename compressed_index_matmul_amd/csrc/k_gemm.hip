// Many-token product y = x dequant(W)^T on bf16 matrix cores (GLQ page,
// "Inference kernels": tensor-core path for batched inputs, decoding codebook
// vectors straight into the matrix operands; the dense W is never written to
// memory).
//
// k_gemm_large -- m > 16.  Tile 256 (tokens) x 128 (W rows), K step 32
//   (4 groups), 4 waves stacked along the tokens, each owning 64 tokens x
//   128 W rows of v_mfma_f32_32x32x16_bf16 accumulators.  Per K step every
//   thread decodes two groups (stage sum and scale in fp32, rounded to bf16)
//   into the LDS W tile, which all four waves read as B fragments; A
//   fragments (x) are loaded from global memory straight into registers.  Tiles are ordered so
//   that consecutive tiles of one token panel land on the same XCD (its L2
//   keeps the x panel).
//
// k_gemm_small -- 1 <= m <= 16 (also vq_gemv with 2..16 bf16 tokens).
//   Persistent workgroups of 8 waves walk 16-row slabs of W; wave w takes
//   every 8th K step; per K step lane l decodes group l/16 of W row l%16
//   directly into its B fragment of v_mfma_f32_16x16x32_bf16 and loads the
//   matching 8 x values of token l%16 as its A fragment.  The eight wave
//   partials are added in LDS in a fixed order.
//
// k_gemm_few (1..64 tokens), k_gemm_tile and k_gemm_wide (many tokens, K %
// 256 == 0) are the tuned kernels for codebooks held in LDS; all kernel
// templates are in gemm_kernels.h.  This file dispatches the plain formats
// (every stage of one width, no stage scales) and the general path of
// residual ladders; ladders with tuned instantiations are dispatched from
// k_gemm_ladder.hip first.
#include <mutex>

#include "gemm_kernels.h"

namespace vqmm {

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <int S, int B>
using UniformLadder = Ladder<B, (S > 1 ? B : 0), (S > 2 ? B : 0), (S > 3 ? B : 0)>;

template <int S, int BITS, bool CB_LDS>
static void launch_gemm_sb(const GemmArgs &a0, hipStream_t s) {
  GemmArgs a = a0;
  if constexpr (CB_LDS && BITS != 16) {
    // 1..64 tokens: the unit kernel (whole eight-step trips per K part, one
    // scale per 128 columns at most)
    if (a.m <= 64 && a.k % 256 == 0 && a.bs % 128 == 0 && a.k < (1 << 20)) {
      if (launch_few<UniformLadder<S, BITS>, false>(a, s)) return;
    }
  }
  if (a.m <= 16) {
    const int nslabs = (a.n + 15) / 16;
    int nwg = device_cu_count();
    if (nwg > nslabs) nwg = nslabs;
    if (a.k % 128 == 0 && a.bs % 32 == 0)
      hipLaunchKernelGGL((k_gemm_small<S, BITS, CB_LDS>), dim3(nwg), dim3(kSWaves * 64), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm_small_gen<S, BITS, CB_LDS>), dim3(nwg), dim3(kSWaves * 64), 0, s, a);
  } else {
    a.tiles_m = (a.m + kLM - 1) / kLM;
    a.tiles_n = (a.n + kLN - 1) / kLN;
    a.per_xcd = (a.tiles_m * a.tiles_n + 7) / 8;
    // buffer paths: K % 32 == 0 and scale blocks of whole K steps (the
    // scale-block multiply is exact for K < 2^20); the 16x16 tile kernels
    // also need K % 256 == 0 and LDS codebooks of 8/12-bit indices
    const bool buf_ok = a.k % 32 == 0 && a.bs % 32 == 0 && a.k < (1 << 20);
    if constexpr (CB_LDS && BITS != 16) {
      if (launch_tiles<UniformLadder<S, BITS>, false>(a, s)) return;
    }
    if (buf_ok)
      hipLaunchKernelGGL((k_gemm_large<S, BITS, CB_LDS, true>), dim3(8 * a.per_xcd), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm_large<S, BITS, CB_LDS, false>), dim3(8 * a.per_xcd), dim3(256), 0, s, a);
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

// Residual ladders of per-stage widths and stage scales (BITS = 0): the
// general slab kernel for 1..16 tokens, the 256 x 128 tile kernel on its
// unaligned path above; codebooks in LDS when every stage fits (no 16-bit
// stage, at most 128 KiB together).
template <int S, bool CB_LDS>
static void launch_gemm_ladder_s(const GemmArgs &a0, hipStream_t s) {
  GemmArgs a = a0;
  if (a.m <= 16) {
    const int nslabs = (a.n + 15) / 16;
    int nwg = device_cu_count();
    if (nwg > nslabs) nwg = nslabs;
    hipLaunchKernelGGL((k_gemm_small_gen<S, 0, CB_LDS>), dim3(nwg), dim3(kSWaves * 64), 0, s, a);
  } else {
    a.tiles_m = (a.m + kLM - 1) / kLM;
    a.tiles_n = (a.n + kLN - 1) / kLN;
    a.per_xcd = (a.tiles_m * a.tiles_n + 7) / 8;
    hipLaunchKernelGGL((k_gemm_large<S, 0, CB_LDS, false>), dim3(8 * a.per_xcd), dim3(256), 0, s, a);
  }
}

template <bool CB_LDS>
static void launch_gemm_ladder(const WView &w, const GemmArgs &a, hipStream_t s) {
  switch (w.S) {
    case 1: launch_gemm_ladder_s<1, CB_LDS>(a, s); break;
    case 2: launch_gemm_ladder_s<2, CB_LDS>(a, s); break;
    case 3: launch_gemm_ladder_s<3, CB_LDS>(a, s); break;
    default: launch_gemm_ladder_s<4, CB_LDS>(a, s); break;
  }
}

// ---------------------------------------------------------------------------
// fp16 path of the 256-token tile kernels
// ---------------------------------------------------------------------------
// x (bf16 [m][k]) -> fp16 after a power-of-two rescale per token that puts
// the token's largest |x| in [2^14, 2^15) (every value within 2^28 of it is
// then exact), written in the A-fragment order of the 16x16x32 kernels:
// token block b (16 tokens), K step s (32 columns), lane l: 16 bytes at
// ((b (k/32) + s) 64 + l) 16 holding token 16 b + l % 16, columns 32 s +
// 8 (l / 16) .. + 8, so a wave's fragment is one contiguous 1 KiB.  Tokens
// m .. m_pad - 1 are zero.  xf[token] = 2^-e undoes the rescale.  One wave
// per token: the row's largest |x| (fixed-order wave reduction), then the
// conversion (the row is read twice; the second read hits in L2).
__global__ __launch_bounds__(256) void k_x_f16(const uint16_t *x, int m, int m_pad, int k, uint16_t *xh,
                                               float *xf) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);  // wave-uniform
  if (tok >= m_pad) return;
  const int chunks = k / 8;  // 8 columns per 16-byte chunk
  const uint4 *row = reinterpret_cast<const uint4 *>(x + (size_t)min(tok, m - 1) * k);
  float mx = 0.f;
  if (tok < m) {
    for (int c = lane; c < chunks; c += 64) {
      const uint4 v = row[c];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf2f(w4[e] & 0xffffu)), fabsf(bf2f(w4[e] >> 16))));
    }
  }
  // fixed-order maximum over the wave (maxima are exact in any order)
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int e = (mx > 0.f && mx <= 3.0e38f) ? 14 - ilogbf(mx) : 0;
  if (lane == 0) xf[tok] = ldexpf(1.f, -e);
  const size_t steps = (size_t)k / 32;
  const size_t blk = (size_t)(tok / 16) * steps * 64 + (tok % 16);
  uint4 *out = reinterpret_cast<uint4 *>(xh);
  for (int c = lane; c < chunks; c += 64) {
    uint4 o = make_uint4(0u, 0u, 0u, 0u);
    if (tok < m) {
      const uint4 v = row[c];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        h[q] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)ldexpf(bf2f(w4[q] & 0xffffu), e),
                                                  (_Float16)ldexpf(bf2f(w4[q] >> 16), e)});
      o = make_uint4(h[0], h[1], h[2], h[3]);
    }
    out[blk + ((size_t)(c / 4) * 64 + 16 * (c % 4))] = o;
  }
}

// The same conversion with the row held in registers (CPL 16-byte chunks per
// lane, k <= 512 CPL): the row is read once, every load issued before the
// maximum is taken.  Output bit-identical to k_x_f16.
template <int CPL>
__global__ __launch_bounds__(256) void k_x_f16_reg(const uint16_t *x, int m, int m_pad, int k, uint16_t *xh,
                                                   float *xf) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);  // wave-uniform
  if (tok >= m_pad) return;
  const int chunks = k / 8;
  const uint4 *row = reinterpret_cast<const uint4 *>(x + (size_t)min(tok, m - 1) * k);
  uint4 v[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    v[j] = (tok < m && c < chunks) ? row[c] : make_uint4(0u, 0u, 0u, 0u);  // padding tokens: zeros
  }
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf2f(w4[e] & 0xffffu)), fabsf(bf2f(w4[e] >> 16))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int e = (mx > 0.f && mx <= 3.0e38f) ? 14 - ilogbf(mx) : 0;
  if (lane == 0) xf[tok] = ldexpf(1.f, -e);
  const size_t steps = (size_t)k / 32;
  const size_t blk = (size_t)(tok / 16) * steps * 64 + (tok % 16);
  uint4 *out = reinterpret_cast<uint4 *>(xh);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c < chunks) {
      const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        h[q] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)ldexpf(bf2f(w4[q] & 0xffffu), e),
                                                  (_Float16)ldexpf(bf2f(w4[q] >> 16), e)});
      out[blk + ((size_t)(c / 4) * 64 + 16 * (c % 4))] = make_uint4(h[0], h[1], h[2], h[3]);
    }
  }
}

namespace {

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// x -> fp16 in fragment order: rows of up to 8192 columns from registers.
void launch_x_f16(const uint16_t *x, int m, int m_pad, int k, uint16_t *xh, float *xf, hipStream_t s) {
  const dim3 grid(m_pad / 4), block(256);
  if (k <= 4096) hipLaunchKernelGGL(k_x_f16_reg<8>, grid, block, 0, s, x, m, m_pad, k, xh, xf);
  else if (k <= 8192) hipLaunchKernelGGL(k_x_f16_reg<16>, grid, block, 0, s, x, m, m_pad, k, xh, xf);
  else hipLaunchKernelGGL(k_x_f16, grid, block, 0, s, x, m, m_pad, k, xh, xf);
}

// Formats with a 256-token tile kernel of one or two stages (the fp16
// variants exist for these): 8/12-bit one stage, 12+12, 8+8, 12+4, 8+4, with
// or without stage scales.
bool tile_f16_format(const WView &w) {
  if (w.S == 1) return w.sb[0] == 8 || w.sb[0] == 12;
  if (w.S != 2) return false;
  const int b0 = w.sb[0], b1 = w.sb[1];
  return (b0 == 12 && (b1 == 12 || b1 == 4)) || (b0 == 8 && (b1 == 8 || b1 == 4));
}

}  // namespace

// The fp16 tile path: more tokens than the few-token kernel takes, a shape
// the tile kernels take, a format with an fp16 variant, and a padded x whose
// bytes (2 m_pad k) a 32-bit buffer range and offset still cover.
bool gemm_f16_takes(const WView &w, int m) {
  const int64_t m_pad = ((int64_t)m + 15) & ~(int64_t)15;
  return m > 64 && w.k % 256 == 0 && w.bs % 32 == 0 && w.k < (1 << 20) && m_pad * w.k < ((int64_t)1 << 31) &&
         tile_f16_format(w);
}

size_t gemm_workspace_bytes(const WView &w, int m) {
  if (!gemm_f16_takes(w, m)) return 0;
  const size_t m_pad = ((size_t)m + 15) & ~(size_t)15;
  return align256(m_pad * (size_t)w.k * 2) + align256(m_pad * 4);
}

// ---------------------------------------------------------------------------
// The product without caller workspace (vq_gemm_noalloc): the scratch the
// fp16 path needs lives in a static device array, one per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel
// (in host code it stands for a host-side shadow, not a device address): its
// device address is looked up once per device with hipGetSymbolAddress and
// that pointer is what the kernels get.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kGemmScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void *g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];

}  // namespace

hipError_t gemm_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

hipError_t launch_gemm(const WView &w, const uint16_t *x, int m, float *y, void *ws, size_t ws_bytes, hipStream_t s) {
  GemmArgs a = make_gemm_args(w, x, m, y);
  if (gemm_f16_takes(w, m) && ws && ws_bytes >= gemm_workspace_bytes(w, m)) {
    const int m_pad = (m + 15) & ~15;
    uint16_t *xh = static_cast<uint16_t *>(ws);
    float *xf = reinterpret_cast<float *>(static_cast<char *>(ws) + align256((size_t)m_pad * w.k * 2));
    launch_x_f16(x, m, m_pad, w.k, xh, xf, s);
    a.xh = xh;
    a.xf = xf;
    a.m_pad = m_pad;
  }
  if (!plain_format(w)) {
    if (launch_gemm_ladder_lds(w, a, s)) return hipGetLastError();
    bool fits = a.cbrows <= kLadderCbRows;
    for (int t = 0; t < w.S; ++t) fits = fits && w.sb[t] != 16;
    if (fits) launch_gemm_ladder<true>(w, a, s);
    else launch_gemm_ladder<false>(w, a, s);
    return hipGetLastError();
  }
  if (w.bits == 8) launch_gemm_bits<8>(w, a, s);
  else if (w.bits == 12) launch_gemm_bits<12>(w, a, s);
  else launch_gemm_bits<16>(w, a, s);
  return hipGetLastError();
}

}  // namespace vqmm
