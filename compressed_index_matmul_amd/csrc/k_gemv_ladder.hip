// Decode-path product for residual ladders and stage scales on the LDS
// kernel (the kernel itself is in gemv_kernels.h).
//
// Instantiated ladders (the ones the pages name, and the plain formats with
// stage scales):
//   * 12 + 4 bits: orka README quick start, the rvq-12-4 mode (a 12-bit
//     primary and a 4-bit residual stage, 2 bits per weight); 8 + 4 bits
//     likewise;
//   * 1-2 stages of 8 or 12 bits with a residual scale per stage (GLQ page,
//     "Inference kernels": the two-stage call takes an inverse residual
//     scale).
// A 4-bit stage's 16-row codebook occupies one 256-byte LDS row: random
// gathers from it never conflict.  Other ladders run on the general kernel.
#include "gemv_kernels.h"

namespace vqmm {

namespace {

// Stage widths packed 4 bits per stage (width / 4), stage 0 lowest.
constexpr int pack2(int b0, int b1) { return (b0 / 4) | ((b1 / 4) << 4); }

int ladder_code(const WView &w) {
  if (w.S > 2) return -1;
  return pack2(w.sb[0], w.S > 1 ? w.sb[1] : 0);
}

template <bool XF16>
bool launch_one(const WView &w, const GemvArgs &a, int cus, hipStream_t s) {
  const int code = ladder_code(w);
  if (!w.scaled) {
    switch (code) {
      case pack2(12, 4): launch_fast_s<Ladder<12, 4>, false, XF16>(a, cus, s); return true;
      case pack2(8, 4): launch_fast_s<Ladder<8, 4>, false, XF16>(a, cus, s); return true;
      default: return false;
    }
  }
  switch (code) {
    case pack2(12, 0): launch_fast_s<Ladder<12>, true, XF16>(a, cus, s); return true;
    case pack2(8, 0): launch_fast_s<Ladder<8>, true, XF16>(a, cus, s); return true;
    case pack2(12, 12): launch_fast_s<Ladder<12, 12>, true, XF16>(a, cus, s); return true;
    case pack2(8, 8): launch_fast_s<Ladder<8, 8>, true, XF16>(a, cus, s); return true;
    case pack2(12, 4): launch_fast_s<Ladder<12, 4>, true, XF16>(a, cus, s); return true;
    case pack2(8, 4): launch_fast_s<Ladder<8, 4>, true, XF16>(a, cus, s); return true;
    default: return false;
  }
}

}  // namespace

bool launch_gemv_lds_ladder(const WView &w, const GemvArgs &a, bool xf16, int cus, hipStream_t s) {
  return xf16 ? launch_one<true>(w, a, cus, s) : launch_one<false>(w, a, cus, s);
}

bool launch_gemv_tokens_ladder(const WView &w, const GemvArgs &a, int batch, int cus, hipStream_t s) {
  const int code = ladder_code(w);
  if (!w.scaled) {
    switch (code) {
      case pack2(12, 4): return launch_tokens_s<Ladder<12, 4>, false>(a, batch, cus, s);
      case pack2(8, 4): return launch_tokens_s<Ladder<8, 4>, false>(a, batch, cus, s);
      default: return false;
    }
  }
  switch (code) {
    case pack2(12, 12): return launch_tokens_s<Ladder<12, 12>, true>(a, batch, cus, s);
    case pack2(12, 4): return launch_tokens_s<Ladder<12, 4>, true>(a, batch, cus, s);
    default: return false;
  }
}

}  // namespace vqmm
