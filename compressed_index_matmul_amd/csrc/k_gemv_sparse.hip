// Decode-path product for weights with a sparse correction (orka README,
// "How it works": the decoded weight plus a sparse correction): the LDS
// kernel instantiated with the correction fused into each row's sum (the
// rows' CSR ranges are loaded once, each row's first 64 entries travel in
// the row ring with its index planes, x is read from the LDS copy), for the
// plain formats and the instantiated ladders.  Kept apart from the
// instantiations without a correction, whose registers it would cost.
#include "gemv_kernels.h"

namespace vqmm {

bool launch_gemv_lds_sparse(const WView &w, const GemvArgs &a, bool xf16, int cus, hipStream_t s) {
  if (plain_lds_format(w)) {
    if (xf16) launch_lds_plain<true, true>(w, a, cus, s);
    else launch_lds_plain<true, false>(w, a, cus, s);
    return true;
  }
  if (plain_format(w)) return false;
  return xf16 ? launch_lds_ladder<true, true>(w, a, cus, s) : launch_lds_ladder<true, false>(w, a, cus, s);
}

bool launch_gemv_tokens_sparse(const WView &w, const GemvArgs &a, int batch, int cus, hipStream_t s) {
  if (plain_format(w)) return launch_tokens_plain<true>(w, a, batch, cus, s);
  return launch_tokens_ladder<true>(w, a, batch, cus, s);
}

}  // namespace vqmm
