// C ABI of libvqmm: argument validation (host only, before any HIP call),
// dispatch to the kernel launchers, status mapping.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "vqmm_internal.h"

namespace vqmm {

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_width(int b) { return b == 4 || b == 8 || b == 12 || b == 16; }

// Full descriptor check; fills `v` on success.  Touches no device state.
int check_weight(const vq_weight *w, WView *v) {
  if (!w) return VQ_ERR_NULL;
  if (w->n_out < 1 || w->k_in < 8 || (w->k_in % 8) != 0) return VQ_ERR_SHAPE;
  if ((int64_t)w->n_out * w->k_in >= ((int64_t)1 << 31)) return VQ_ERR_SHAPE;
  if (w->n_stages < 1 || w->n_stages > VQ_MAX_STAGES) return VQ_ERR_SHAPE;
  if (w->scale_block < 8 || (w->scale_block % 8) != 0) return VQ_ERR_SHAPE;
  if ((w->flags & ~VQ_STAGE_SCALES) != 0) return VQ_ERR_UNSUPPORTED;
  int sb[VQ_MAX_STAGES];
  for (int t = 0; t < w->n_stages; ++t) {
    sb[t] = w->stage_bits[t] != 0 ? w->stage_bits[t] : w->idx_bits;
    if (!valid_width(sb[t])) return VQ_ERR_UNSUPPORTED;
    if ((w->flags & VQ_STAGE_SCALES) && !std::isfinite(w->stage_scale[t])) return VQ_ERR_VALUE;
  }
  for (int t = 0; t < w->n_stages; ++t) {
    if (!w->codebook[t]) return VQ_ERR_NULL;
    if (!aligned16(w->codebook[t])) return VQ_ERR_ALIGN;
    const bool need16 = sb[t] == 16;
    const bool need_lo = sb[t] == 8 || sb[t] == 12;
    const bool need_hi = sb[t] == 4 || sb[t] == 12;
    if ((need16 && !w->idx16[t]) || (need_lo && !w->idx_lo[t]) || (need_hi && !w->idx_hi[t])) return VQ_ERR_NULL;
    if ((need16 && !aligned16(w->idx16[t])) || (need_lo && !aligned16(w->idx_lo[t])) ||
        (need_hi && !aligned16(w->idx_hi[t])))
      return VQ_ERR_ALIGN;
  }
  if (!w->scales) return VQ_ERR_NULL;
  if (!aligned16(w->scales)) return VQ_ERR_ALIGN;
  if (w->sp_nnz < 0 || w->sp_reserved != 0) return VQ_ERR_SHAPE;
  if (w->sp_nnz > 0) {
    if (!w->sp_rowptr || !w->sp_col || !w->sp_val) return VQ_ERR_NULL;
    if (!aligned16(w->sp_rowptr) || !aligned16(w->sp_col) || !aligned16(w->sp_val)) return VQ_ERR_ALIGN;
  }
  if (w->lr_rank < 0 || w->lr_rank > VQ_MAX_LR_RANK || w->lr_reserved != 0) return VQ_ERR_SHAPE;
  if (w->lr_rank > 0) {
    if (!w->lr_u || !w->lr_v) return VQ_ERR_NULL;
    if (!aligned16(w->lr_u) || !aligned16(w->lr_v)) return VQ_ERR_ALIGN;
    if ((int64_t)w->lr_rank * w->n_out >= ((int64_t)1 << 31) || (int64_t)w->lr_rank * w->k_in >= ((int64_t)1 << 31))
      return VQ_ERR_SHAPE;
  }
  if (v) {
    *v = WView{};
    v->n = w->n_out;
    v->k = w->k_in;
    v->G = w->k_in / 8;
    v->S = w->n_stages;
    v->uniform = true;
    v->scaled = false;
    for (int t = 0; t < VQ_MAX_STAGES; ++t) v->rs[t] = 1.0f;
    for (int t = 0; t < w->n_stages; ++t) {
      v->sb[t] = sb[t];
      v->uniform = v->uniform && sb[t] == sb[0];
      if (w->flags & VQ_STAGE_SCALES) {
        v->rs[t] = w->stage_scale[t];
        v->scaled = v->scaled || w->stage_scale[t] != 1.0f;
      }
    }
    v->bits = v->uniform ? sb[0] : 0;
    v->bs = w->scale_block > w->k_in ? w->k_in : w->scale_block;
    v->nblk = (w->k_in + v->bs - 1) / v->bs;
    for (int t = 0; t < w->n_stages; ++t) {
      v->lo[t] = w->idx_lo[t];
      v->hi[t] = w->idx_hi[t];
      v->i16[t] = w->idx16[t];
      v->cb[t] = w->codebook[t];
    }
    v->sc = w->scales;
    v->sp_nnz = w->sp_nnz;
    v->sp_rowptr = w->sp_nnz > 0 ? w->sp_rowptr : nullptr;
    v->sp_col = w->sp_nnz > 0 ? w->sp_col : nullptr;
    v->sp_val = w->sp_nnz > 0 ? w->sp_val : nullptr;
    v->lr_rank = w->lr_rank;
    v->lr_u = w->lr_rank > 0 ? w->lr_u : nullptr;
    v->lr_v = w->lr_rank > 0 ? w->lr_v : nullptr;
  }
  return VQ_OK;
}

int map_hip(hipError_t e) { return e == hipSuccess ? VQ_OK : VQ_ERR_HIP; }

// Workspace of the many-token product: the main product's part, then the
// low-rank correction's t (both 256-byte multiples).
size_t total_workspace_bytes(const WView &v, int m) { return gemm_workspace_bytes(v, m) + lowrank_workspace_bytes(v, m); }

// Grid limit of the low-rank kernels for many tokens (64-token tiles in
// grid.y).
bool lowrank_rows_fit(const WView &v, int m) { return v.lr_rank == 0 || (m + 63) / 64 <= 65535; }

// The many-token product with its corrections; ws holds at least
// total_workspace_bytes(v, m) bytes (null when that is 0).
int run_gemm(const WView &v, const uint16_t *x, int m, float *y, void *ws, hipStream_t s) {
  const size_t main_bytes = gemm_workspace_bytes(v, m);
  int st = map_hip(launch_gemm(v, x, m, y, main_bytes > 0 ? ws : nullptr, main_bytes, s));
  if (st != VQ_OK) return st;
  st = map_hip(launch_sparse_add(v, x, VQ_BF16, m, y, s));
  if (st != VQ_OK || v.lr_rank == 0) return st;
  float *t = reinterpret_cast<float *>(static_cast<char *>(ws) + main_bytes);
  return map_hip(launch_lowrank_gemm(v, x, m, y, t, s));
}

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev] = n;
  });
  return g_cu_count[dev];
}

}  // namespace vqmm

using namespace vqmm;

extern "C" {

int vq_version(void) { return VQMM_VERSION; }

const char *vq_status_string(int status) {
  switch (status) {
    case VQ_OK: return "ok";
    case VQ_ERR_NULL: return "a required pointer is NULL";
    case VQ_ERR_SHAPE: return "a size is out of range or inconsistent";
    case VQ_ERR_DTYPE: return "unsupported element type";
    case VQ_ERR_UNSUPPORTED: return "request outside what the kernels implement";
    case VQ_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case VQ_ERR_HIP: return "HIP runtime error";
    case VQ_ERR_VALUE: return "a scalar argument value is invalid";
    case VQ_ERR_WORKSPACE: return "the workspace is smaller than vq_gemm_workspace_size";
    default: return "unknown status";
  }
}

int vq_validate(const vq_weight *w) { return check_weight(w, nullptr); }

int64_t vq_compressed_bytes(const vq_weight *w) {
  WView v;
  const int st = check_weight(w, &v);
  if (st != VQ_OK) return st;
  const int64_t groups = (int64_t)v.n * v.G;
  int64_t total = 2 * (int64_t)v.n * v.nblk;
  for (int t = 0; t < v.S; ++t) {
    const int b = v.sb[t];
    total += b == 16 ? 2 * groups : b == 12 ? groups + (groups + 1) / 2 : b == 8 ? groups : (groups + 1) / 2;
    total += ((int64_t)1 << b) * 16;
  }
  if (v.sp_nnz > 0) total += 4 * ((int64_t)v.n + 1) + 6 * (int64_t)v.sp_nnz;
  if (v.lr_rank > 0) total += 2 * (int64_t)v.lr_rank * ((int64_t)v.n + v.k);
  return total;
}

int vq_unpack_dequant(const vq_weight *w, uint16_t *idx_out, uint16_t *w_out, void *stream) {
  WView v;
  int st = check_weight(w, &v);
  if (st != VQ_OK) return st;
  if (!idx_out && !w_out) return VQ_ERR_NULL;
  if ((idx_out && !aligned16(idx_out)) || (w_out && !aligned16(w_out))) return VQ_ERR_ALIGN;
  return map_hip(launch_unpack_dequant(v, idx_out, w_out, reinterpret_cast<hipStream_t>(stream)));
}

int vq_gemv(const vq_weight *w, const void *x, int32_t x_dtype, int32_t batch, float *y, void *stream) {
  WView v;
  int st = check_weight(w, &v);
  if (st != VQ_OK) return st;
  if (!x || !y) return VQ_ERR_NULL;
  if (x_dtype != VQ_F32 && x_dtype != VQ_BF16) return VQ_ERR_DTYPE;
  if (batch < 1 || batch > 16) return VQ_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y)) return VQ_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  bool sp_done = false;  // the sparse correction was added by the product kernel
  if (batch > 1 && x_dtype == VQ_BF16) {
    hipError_t e = hipSuccess;
    if (launch_gemv_tokens(v, x, batch, y, s, &e)) sp_done = true;
    else e = launch_gemm(v, reinterpret_cast<const uint16_t *>(x), batch, y, nullptr, 0, s);
    if (e != hipSuccess) return VQ_ERR_HIP;
  } else {
    const size_t esz = x_dtype == VQ_F32 ? 4 : 2;
    for (int b = 0; b < batch; ++b) {
      const void *xb = reinterpret_cast<const char *>(x) + (size_t)b * v.k * esz;
      st = map_hip(launch_gemv_token(v, xb, x_dtype, y + (size_t)b * v.n, s, &sp_done));
      if (st != VQ_OK) return st;
    }
  }
  if (!sp_done) {
    st = map_hip(launch_sparse_add(v, x, x_dtype, batch, y, s));
    if (st != VQ_OK) return st;
  }
  return map_hip(launch_lowrank_tokens(v, x, x_dtype, batch, y, s));
}

int vq_gemm(const vq_weight *w, const uint16_t *x_bf16, int32_t m, float *y, void *workspace, size_t ws_bytes,
            void *stream) {
  WView v;
  int st = check_weight(w, &v);
  if (st != VQ_OK) return st;
  if (!x_bf16 || !y) return VQ_ERR_NULL;
  if (m < 1) return VQ_ERR_SHAPE;
  if ((int64_t)m * v.k >= ((int64_t)1 << 31) || (int64_t)m * v.n >= ((int64_t)1 << 31)) return VQ_ERR_SHAPE;
  if (ws_bytes > 0 && !workspace) return VQ_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(y) || !aligned16(workspace)) return VQ_ERR_ALIGN;
  if (!lowrank_rows_fit(v, m)) return VQ_ERR_UNSUPPORTED;
  if (ws_bytes < total_workspace_bytes(v, m)) return VQ_ERR_WORKSPACE;
  return run_gemm(v, x_bf16, m, y, workspace, reinterpret_cast<hipStream_t>(stream));
}

int vq_gemm_noalloc(const vq_weight *w, const uint16_t *x_bf16, int32_t m, float *y, void *stream) {
  WView v;
  int st = check_weight(w, &v);
  if (st != VQ_OK) return st;
  if (!x_bf16 || !y) return VQ_ERR_NULL;
  if (m < 1) return VQ_ERR_SHAPE;
  if ((int64_t)m * v.k >= ((int64_t)1 << 31) || (int64_t)m * v.n >= ((int64_t)1 << 31)) return VQ_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(y)) return VQ_ERR_ALIGN;
  if (!lowrank_rows_fit(v, m)) return VQ_ERR_UNSUPPORTED;
  const size_t need = total_workspace_bytes(v, m);
  if (need > kGemmScratchBytes) return VQ_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need > 0 && gemm_scratch(&ws) != hipSuccess) return VQ_ERR_HIP;
  return run_gemm(v, x_bf16, m, y, ws, reinterpret_cast<hipStream_t>(stream));
}

size_t vq_gemm_workspace_size(const vq_weight *w, int32_t m) {
  WView v;
  if (check_weight(w, &v) != VQ_OK || m < 1) return 0;
  if ((int64_t)m * v.k >= ((int64_t)1 << 31) || (int64_t)m * v.n >= ((int64_t)1 << 31)) return 0;
  return total_workspace_bytes(v, m);
}

int vq_gemv_rht(const vq_weight *w, const void *x, int32_t x_dtype, int32_t batch, const int8_t *signs,
                int32_t max_block, float *y, void *stream) {
  WView v;
  int st = check_weight(w, &v);
  if (st != VQ_OK) return st;
  if (!x || !signs || !y) return VQ_ERR_NULL;
  if (x_dtype != VQ_F32 && x_dtype != VQ_BF16) return VQ_ERR_DTYPE;
  if (batch < 1 || batch > 16) return VQ_ERR_UNSUPPORTED;
  if (max_block < 1 || max_block > 16384 || (max_block & (max_block - 1)) != 0) return VQ_ERR_SHAPE;
  if (!gemv_rht_takes(v)) return VQ_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(signs) || !aligned16(y)) return VQ_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t esz = x_dtype == VQ_F32 ? 4 : 2;
  for (int b = 0; b < batch; ++b) {
    const void *xb = reinterpret_cast<const char *>(x) + (size_t)b * v.k * esz;
    st = map_hip(launch_gemv_rht_token(v, xb, x_dtype, signs, max_block, y + (size_t)b * v.n, s));
    if (st != VQ_OK) return st;
  }
  return VQ_OK;
}

static_assert(VQ_RHT_MAX_SHARDS == kRhtMaxShards, "shard limit of the header and the kernels");

int rht_apply(const void *x, int32_t x_dtype, int32_t batch, int32_t n, const int8_t *signs,
              int32_t max_block, float *out, void *stream) {
  return rht_apply_shards(x, x_dtype, batch, n, 1, &n, signs, max_block, VQ_RHT_FORWARD, out, stream);
}

int rht_apply_shards(const void *x, int32_t x_dtype, int32_t batch, int32_t n, int32_t n_shards,
                     const int32_t *shard_len, const int8_t *signs, int32_t max_block, int32_t direction,
                     float *out, void *stream) {
  if (!x || !signs || !out || !shard_len) return VQ_ERR_NULL;
  if (x_dtype != VQ_F32 && x_dtype != VQ_BF16) return VQ_ERR_DTYPE;
  if (direction != VQ_RHT_FORWARD && direction != VQ_RHT_INVERSE) return VQ_ERR_VALUE;
  if (batch < 1 || n < 1 || n_shards < 1 || n_shards > VQ_RHT_MAX_SHARDS) return VQ_ERR_SHAPE;
  if (max_block < 1 || max_block > 16384 || (max_block & (max_block - 1)) != 0) return VQ_ERR_SHAPE;
  int64_t total = 0;
  for (int i = 0; i < n_shards; ++i) {
    if (shard_len[i] < 1) return VQ_ERR_SHAPE;
    total += shard_len[i];
  }
  if (total != n) return VQ_ERR_SHAPE;
  if ((int64_t)batch * n >= ((int64_t)1 << 31)) return VQ_ERR_SHAPE;
  if ((int64_t)rht_grid_blocks(n_shards, shard_len, max_block) * batch >= ((int64_t)1 << 31)) return VQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(out)) return VQ_ERR_ALIGN;
  return map_hip(launch_rht(x, x_dtype, batch, n, n_shards, shard_len, signs, max_block,
                            direction == VQ_RHT_INVERSE, out, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
