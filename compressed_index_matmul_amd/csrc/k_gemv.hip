// Decode-path product y = x dequant(W)^T for one token (GLQ page, "Inference
// kernels": each output row walks its K/8 codebook groups, gathering 8-wide
// codebook vectors, and accumulates against the indices without forming W;
// split-K-style lane partials reduced inside the wave in a fixed order).
//
// k_gemv_lds  -- codebooks and x that fit in one workgroup's LDS (8/12-bit,
//                K % 32 == 0, scale_block % 32 == 0; K <= 16384 for bf16 x).
//   * persistent grid, one workgroup per CU holding a contiguous block of
//     rows; its waves take every WAVES-th row of the block;
//   * prologue: x loads, the first rows' index loads (HBM) and the codebooks
//     (LDS-direct, global_load_lds_dwordx4) are all in flight together; x is
//     converted once per workgroup into LDS;
//   * lane l owns the 4-group chunks c = l + 64 j of every row; per chunk and
//     stage it loads one dword of the low-byte plane and one short of the
//     high-nibble plane (coalesced 256 B + 128 B per wave); a ring of row
//     buffers keeps the next rows' loads in flight while a row is computed;
//   * bf16 x is held as fp16 after a per-chunk power-of-two rescale (exact
//     for values within 2^28 of the chunk's largest |x|), so a group-stage
//     costs one 16-byte LDS gather and four v_dot2_f32_f16; fp32 x uses fma;
//   * the lane partial is scaled per chunk (block scale times the inverse
//     rescale) and summed across the wave with DPP (fixed order, no atomics).
//
// k_gemv_gen  -- everything else (16-bit indices into a 1 MiB codebook, 3-4
//                12-bit stages, ragged K or scale blocks, ladders without an
//                LDS kernel of their own): codebook rows are gathered from
//                global memory (L2-resident), x is staged in LDS as fp32,
//                one wave per row, lane = 4 consecutive groups when
//                K % 32 == 0, else one group.
//
// Residual ladders (mixed per-stage widths, GLQ page "Bit widths"; orka's
// rvq-12-4) and stage scales (GLQ page, "Inference kernels": the inverse
// residual scale of the two-stage call) run on k_gemv_lds instantiated for
// the ladder in k_gemv_ladder.hip when every codebook fits in LDS, else on
// k_gemv_gen with the widths and scales read at run time.
#include "gemv_kernels.h"

namespace vqmm {

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
// Codebook rows of every stage when all of them can sit in LDS (no 16-bit
// stage), else 0.
static int lds_codebook_rows(const WView &w) {
  int rows = 0;
  for (int t = 0; t < w.S; ++t) {
    if (w.sb[t] == 16) return 0;
    rows += 1 << w.sb[t];
  }
  return rows;
}

// x is staged in LDS; the fast path needs the codebooks and x of a whole row
// in one workgroup's LDS, up to 8 chunks per lane (K <= 16384) for bf16 x and
// 4 for fp32 x (held in registers).
static bool gemv_fast_shape(const WView &w, int xt) {
  const int rows = lds_codebook_rows(w);
  if (rows == 0) return false;
  if (w.k % 32 || w.bs % 32) return false;
  const int cpl = (w.G / 4 + 63) / 64;
  if (cpl > (xt == VQ_BF16 ? 8 : 4)) return false;
  return gemv_lds_bytes(rows, cpl, xt == VQ_BF16) <= kLdsBytes;
}

// The general kernel: BITS = the width of every stage of a plain format, 0
// for ladders and stage scales.
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

bool launch_gemv_tokens(const WView &w, const void *x, int batch, float *y, hipStream_t s, hipError_t *err) {
  if (batch < 2 || batch > 4 || !gemv_fast_shape(w, VQ_BF16)) return false;
  if ((w.G / 4 + 63) / 64 > 3) return false;
  GemvArgs a = make_args(w);
  a.x = x;
  a.y = y;
  const int cus = device_cu_count();
  bool done = false;
  if (w.sp_nnz > 0) done = launch_gemv_tokens_sparse(w, a, batch, cus, s);
  else if (!plain_format(w)) done = launch_gemv_tokens_ladder(w, a, batch, cus, s);
  else done = launch_tokens_plain<false>(w, a, batch, cus, s);
  if (done) *err = hipGetLastError();
  return done;
}

hipError_t launch_gemv_token(const WView &w, const void *x, int xt, float *y, hipStream_t s, bool *sp_done) {
  GemvArgs a = make_args(w);
  a.x = x;
  a.y = y;
  const int cus = device_cu_count();
  const bool xf16 = xt == VQ_BF16;
  // the LDS kernel adds a sparse correction itself
  *sp_done = true;
  if (gemv_fast_shape(w, xt)) {
    if (w.sp_nnz > 0) {
      if (launch_gemv_lds_sparse(w, a, xf16, cus, s)) return hipGetLastError();
    } else if (plain_lds_format(w)) {
      if (xf16) launch_lds_plain<false, true>(w, a, cus, s);
      else launch_lds_plain<false, false>(w, a, cus, s);
      return hipGetLastError();
    } else if (!plain_format(w) && launch_gemv_lds_ladder(w, a, xf16, cus, s)) {
      return hipGetLastError();
    }
  }
  *sp_done = false;
  if (launch_gemv_cbs(w, x, xt, y, cus, s)) return hipGetLastError();
  if (launch_gemv_l2(w, a, xt, cus, s)) return hipGetLastError();
  if (!plain_format(w)) launch_gen_bits<0>(w, a, xt, cus, s);
  else if (w.bits == 8) launch_gen_bits<8>(w, a, xt, cus, s);
  else if (w.bits == 12) launch_gen_bits<12>(w, a, xt, cus, s);
  else launch_gen_bits<16>(w, a, xt, cus, s);
  return hipGetLastError();
}

bool gemv_rht_takes(const WView &w) {
  return w.sp_nnz == 0 && w.lr_rank == 0 && (gemv_cbs_rht_takes(w) || gemv_l2_takes(w));
}

hipError_t launch_gemv_rht_token(const WView &w, const void *x, int xt, const int8_t *signs, int max_block, float *y,
                                 hipStream_t s) {
  const int cus = device_cu_count();
  if (launch_gemv_cbs(w, x, xt, y, cus, s, signs, max_block)) return hipGetLastError();
  GemvArgs a = make_args(w);
  a.x = x;
  a.y = y;
  if (!launch_gemv_l2(w, a, xt, cus, s, signs, max_block)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vqmm
