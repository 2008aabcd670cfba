// Internal interface between the C-ABI layer (vqmm_api.cpp) and the kernel
// launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/vqmm.h"

namespace vqmm {

// Validated, flattened view of a vq_weight.
struct WView {
  int n;      // n_out
  int k;      // k_in
  int G;      // groups per row = k / 8
  int S;      // stages
  int bits;   // index width of every stage when `uniform`, else 0
  int sb[VQ_MAX_STAGES];  // index width of each stage: 4, 8, 12 or 16
  bool uniform;           // every stage has the same width
  bool scaled;            // some stage scale differs from 1
  float rs[VQ_MAX_STAGES];  // stage scales (1 without VQ_STAGE_SCALES)
  int bs;     // scale_block (clamped to k when larger)
  int nblk;   // scales per row
  const uint8_t *lo[VQ_MAX_STAGES];
  const uint8_t *hi[VQ_MAX_STAGES];
  const uint16_t *i16[VQ_MAX_STAGES];
  const uint16_t *cb[VQ_MAX_STAGES];
  const uint16_t *sc;
  int sp_nnz;              // sparse correction entries (0: none)
  const int32_t *sp_rowptr;
  const int32_t *sp_col;
  const uint16_t *sp_val;
  int lr_rank;             // low-rank correction rank (0: none)
  const uint16_t *lr_u;    // fp16 [n][lr_rank]
  const uint16_t *lr_v;    // fp16 [lr_rank][k]
};

// The plain formats the specialised kernels take: every stage of one width
// (8, 12 or 16 bits) and no stage scales.
inline bool plain_format(const WView &w) { return w.uniform && !w.scaled && w.bits >= 8; }

// Compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_unpack_dequant(const WView &w, uint16_t *idx_out, uint16_t *w_out, hipStream_t s);
// Shards per row of one transform launch.
constexpr int kRhtMaxShards = 16;
// grid.x workgroups per token of a transform launch: the most blocks of any
// shard.
int rht_grid_blocks(int nsh, const int32_t *shard_len, int max_block);
// The transform of batch rows of n = sum(shard_len) columns, each shard on
// its own; forward = signs then Hadamard, inverse = Hadamard then signs.
hipError_t launch_rht(const void *x, int xt, int batch, int n, int nsh, const int32_t *shard_len,
                      const int8_t *signs, int max_block, bool inverse, float *out, hipStream_t s);
// One token of x (fp32 or bf16, VQ_F32 / VQ_BF16) against W: y[n].
// *sp_done: the launched kernel also added the sparse correction.
hipError_t launch_gemv_token(const WView &w, const void *x, int xt, float *y, hipStream_t s, bool *sp_done);
// The product with the input transform applied inside the decode kernel:
// whether the weight has such a kernel (a 16-bit weight the sliced or the
// L2 decode kernel takes, no sparse or low-rank correction), and one token's
// launch.
bool gemv_rht_takes(const WView &w);
hipError_t launch_gemv_rht_token(const WView &w, const void *x, int xt, const int8_t *signs, int max_block, float *y,
                                 hipStream_t s);
// 2..4 bf16 tokens in one launch of the LDS decode kernel when the shape
// allows it (false: not taken, nothing launched; *err set when taken).  The
// kernel also adds the sparse correction.
bool launch_gemv_tokens(const WView &w, const void *x, int batch, float *y, hipStream_t s, hipError_t *err);
// The many-token product; ws / ws_bytes: the caller's workspace (may be
// null / 0), at least gemm_workspace_bytes(w, m) bytes.
hipError_t launch_gemm(const WView &w, const uint16_t *x, int m, float *y, void *ws, size_t ws_bytes, hipStream_t s);
// Workspace bytes the many-token product of m tokens needs (0: none).
size_t gemm_workspace_bytes(const WView &w, int m);
// The library's own scratch for vq_gemm_noalloc: kGemmScratchBytes of device
// memory per GPU (a static device array), its address on the current device.
constexpr size_t kGemmScratchBytes = (size_t)33 << 20;
hipError_t gemm_scratch(void **ptr);
// y[b][r] += sum_j val_j x[b][col_j] over the sparse correction's row r, for
// m tokens of x (VQ_F32 / VQ_BF16); after the main product on the same
// stream.  No-op without a correction.
hipError_t launch_sparse_add(const WView &w, const void *x, int xt, int m, float *y, hipStream_t s);
// The low-rank correction's term y += (x V^T) U^T, after the main product on
// the same stream; no-op without one.  Tokens (1..16, VQ_F32 / VQ_BF16):
// one launch, no scratch.  Many bf16 tokens: t [m][lr_rank] in the caller's
// workspace (lowrank_workspace_bytes), two launches.
hipError_t launch_lowrank_tokens(const WView &w, const void *x, int xt, int batch, float *y, hipStream_t s);
size_t lowrank_workspace_bytes(const WView &w, int m);
hipError_t launch_lowrank_gemm(const WView &w, const uint16_t *x, int m, float *y, float *t, hipStream_t s);


}  // namespace vqmm
