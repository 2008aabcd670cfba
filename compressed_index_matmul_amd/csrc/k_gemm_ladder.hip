// Many-token product for residual ladders and stage scales on the tuned
// matrix-core kernels (k_gemm_few for 1..64 tokens, k_gemm_tile /
// k_gemm_wide for more; templates in gemm_kernels.h).
//
// Instantiated ladders, as for the decode kernel: 12 + 4 and 8 + 4 bits
// (orka README quick start, the rvq-12-4 mode), and 1-2 stages of 8 or 12
// bits with a residual scale per stage (GLQ page, "Inference kernels": the
// inverse residual scale of the two-stage call).  Other ladders, and shapes
// these kernels do not take, run on the general kernels of k_gemm.hip.
#include "gemm_kernels.h"

namespace vqmm {

namespace {

// Stage widths packed 4 bits per stage (width / 4), stage 0 lowest.
constexpr int pack2(int b0, int b1) { return (b0 / 4) | ((b1 / 4) << 4); }

template <class LD, bool RS>
bool launch_lds(const GemmArgs &a0, hipStream_t s) {
  GemmArgs a = a0;
  if (a.m <= 64 && a.k % 256 == 0 && a.bs % 128 == 0 && a.k < (1 << 20)) {
    if (launch_few<LD, RS>(a, s)) return true;
  }
  if (a.m <= 16) return false;
  a.tiles_m = (a.m + kLM - 1) / kLM;
  a.tiles_n = (a.n + kLN - 1) / kLN;
  a.per_xcd = (a.tiles_m * a.tiles_n + 7) / 8;
  return launch_tiles<LD, RS>(a, s);
}

}  // namespace

bool launch_gemm_ladder_lds(const WView &w, const GemmArgs &a, hipStream_t s) {
  if (w.S > 2) return false;
  const int code = pack2(w.sb[0], w.S > 1 ? w.sb[1] : 0);
  if (!w.scaled) {
    switch (code) {
      case pack2(12, 4): return launch_lds<Ladder<12, 4>, false>(a, s);
      case pack2(8, 4): return launch_lds<Ladder<8, 4>, false>(a, s);
      default: return false;
    }
  }
  switch (code) {
    case pack2(12, 0): return launch_lds<Ladder<12>, true>(a, s);
    case pack2(8, 0): return launch_lds<Ladder<8>, true>(a, s);
    case pack2(12, 12): return launch_lds<Ladder<12, 12>, true>(a, s);
    case pack2(8, 8): return launch_lds<Ladder<8, 8>, true>(a, s);
    case pack2(12, 4): return launch_lds<Ladder<12, 4>, true>(a, s);
    case pack2(8, 4): return launch_lds<Ladder<8, 4>, true>(a, s);
    default: return false;
  }
}

}  // namespace vqmm
