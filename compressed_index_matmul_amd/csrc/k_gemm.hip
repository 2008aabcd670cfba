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

size_t gemm_workspace_bytes(const WView &w, int m) {
  (void)w;
  (void)m;
  return 0;  // no kernel of the many-token product keeps scratch
}

hipError_t launch_gemm(const WView &w, const uint16_t *x, int m, float *y, void *ws, size_t ws_bytes, hipStream_t s) {
  (void)ws;
  (void)ws_bytes;
  const GemmArgs a = make_gemm_args(w, x, m, y);
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
