// Decode-path product for residual ladders and stage scales on the LDS
// kernel (kernel and format dispatch in gemv_kernels.h): the instantiations
// without a sparse correction.
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

bool launch_gemv_lds_ladder(const WView &w, const GemvArgs &a, bool xf16, int cus, hipStream_t s) {
  return xf16 ? launch_lds_ladder<false, true>(w, a, cus, s) : launch_lds_ladder<false, false>(w, a, cus, s);
}

bool launch_gemv_tokens_ladder(const WView &w, const GemvArgs &a, int batch, int cus, hipStream_t s) {
  return launch_tokens_ladder<false>(w, a, batch, cus, s);
}

}  // namespace vqmm
