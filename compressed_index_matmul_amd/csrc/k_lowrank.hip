// Low-rank correction of the decoded weight (orka README, CLI: the correct
// command adds a low-rank or sparse correction; the form W += U V with fp16
// factors U [n][r], V [r][k] is this library's reading).  The products never
// form U V: they take t = x V^T, then y += t U^T, both in fp32 with a fixed
// order, after the main product on the same stream.
//
// Decode (1..16 tokens, no scratch): k_lr_tokens.  Every workgroup forms
// the whole t for all tokens itself -- waves own rows j of V, lanes own 8
// columns of a 512-column chunk of x staged in LDS, a lane's partial runs
// over the chunks in order and one fixed-order wave reduction gives t[b][j]
// -- then adds t U^T to its own range of output rows.  The grid is sized so
// that the repeated t (r k b multiply-adds and one read of V per workgroup,
// from L2) stays small next to the rows' work.
//
// Many tokens (the caller's workspace holds t): k_lr_mm, a plain LDS-tiled
// fp32 product C (+)= A B^T used twice, t = x V^T and y += t U^T; each
// output's sum runs over the inner index in order.
#include "vqmm_device.h"
#include "vqmm_internal.h"

namespace vqmm {

namespace {

constexpr int kLrThreads = 512;  // eight waves
constexpr int kLrWaves = kLrThreads / 64;
constexpr int kLrChunk = 512;    // columns of x per staging step: 8 per lane
constexpr int kLrMaxTok = 16;

struct LrTokArgs {
  const void *x;      // [B][k], fp32 or bf16
  const uint16_t *u;  // fp16 [n][r]
  const uint16_t *v;  // fp16 [r][k]
  float *y;           // [B][n], added to
  int B, k, r, n;
  int rows_per_wg;
};

// BT: the most tokens of the instance (B <= BT); JB: rows of V per wave and
// round (JB * BT accumulators per lane).
template <bool BF16, int BT, int JB>
__global__ __launch_bounds__(kLrThreads) void k_lr_tokens(LrTokArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[BT][kLrChunk];
  __shared__ float ts[BT][VQ_MAX_LR_RANK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = a.B;

  // t = x V^T for every token, rounds of kLrWaves * JB rows of V
  for (int jr = 0; jr < a.r; jr += kLrWaves * JB) {
    const int j0 = jr + wave * JB;  // wave-uniform
    float acc[JB][BT];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[jj][b] = 0.f;
    for (int c0 = 0; c0 < a.k; c0 += kLrChunk) {
      __syncthreads();  // every wave is done with the previous chunk
      for (int e = tid; e < B * kLrChunk; e += kLrThreads) {
        const int b = e / kLrChunk, c = e % kLrChunk;
        float v = 0.f;
        if (c0 + c < a.k) {
          const int64_t i = (int64_t)b * a.k + c0 + c;
          v = BF16 ? bf2f(reinterpret_cast<const uint16_t *>(a.x)[i]) : reinterpret_cast<const float *>(a.x)[i];
        }
        xs[b][c] = v;
      }
      __syncthreads();
      const int c = c0 + 8 * lane;
      if (c < a.k) {  // k % 8 == 0: a lane's 8 columns are all in or all out
        float xv[BT][8];
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b < B) {
            const float4 p = *reinterpret_cast<const float4 *>(&xs[b][8 * lane]);
            const float4 q = *reinterpret_cast<const float4 *>(&xs[b][8 * lane + 4]);
            xv[b][0] = p.x, xv[b][1] = p.y, xv[b][2] = p.z, xv[b][3] = p.w;
            xv[b][4] = q.x, xv[b][5] = q.y, xv[b][6] = q.z, xv[b][7] = q.w;
          }
        }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          const int j = j0 + jj;
          if (j < a.r) {  // wave-uniform
            const uint4 h = *reinterpret_cast<const uint4 *>(a.v + (int64_t)j * a.k + c);
            const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
            float vf[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) vf[q] = h2f((hw[q >> 1] >> (16 * (q & 1))) & 0xffffu);
#pragma unroll
            for (int b = 0; b < BT; ++b) {
              if (b < B) {
                float s = acc[jj][b];
#pragma unroll
                for (int q = 0; q < 8; ++q) s = fmaf(vf[q], xv[b][q], s);
                acc[jj][b] = s;
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int j = j0 + jj;
      if (j < a.r) {
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b < B) {
            const float s = wave_sum(acc[jj][b]);
            if (lane == 0) ts[b][j] = s;
          }
        }
      }
    }
  }
  __syncthreads();

  // y[b][i] += sum_j U[i][j] t[b][j] over this workgroup's rows
  const int r0 = blockIdx.x * a.rows_per_wg;
  const int r1 = min(r0 + a.rows_per_wg, a.n);
  for (int i = r0 + tid; i < r1; i += kLrThreads) {
    float s[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) s[b] = 0.f;
    const uint16_t *ur = a.u + (int64_t)i * a.r;
    for (int j = 0; j < a.r; ++j) {
      const float u = h2f(ur[j]);
#pragma unroll
      for (int b = 0; b < BT; ++b)
        if (b < B) s[b] = fmaf(u, ts[b][j], s[b]);
    }
#pragma unroll
    for (int b = 0; b < BT; ++b)
      if (b < B) a.y[(int64_t)b * a.n + i] += s[b];
  }
}

template <bool BF16>
void launch_tokens_dt(const LrTokArgs &a, int grid, hipStream_t s) {
  if (a.B <= 1) hipLaunchKernelGGL((k_lr_tokens<BF16, 1, 8>), dim3(grid), dim3(kLrThreads), 0, s, a);
  else if (a.B <= 4) hipLaunchKernelGGL((k_lr_tokens<BF16, 4, 4>), dim3(grid), dim3(kLrThreads), 0, s, a);
  else hipLaunchKernelGGL((k_lr_tokens<BF16, 16, 2>), dim3(grid), dim3(kLrThreads), 0, s, a);
}

// C[m][n] (+)= sum_k A[m][k] B[n][k]: A fp32 or bf16 bits, B fp16 bits, C
// fp32, all row-major with row pitch = the inner size.  64 x 64 outputs per
// workgroup, 4 x 4 per thread, inner steps of 16 through LDS.
constexpr int kMmTile = 64;
constexpr int kMmStep = 16;

struct LrMmArgs {
  const void *a;
  const uint16_t *b;
  float *c;
  int M, N, K;
};

template <bool ABF16, bool ACC>
__global__ __launch_bounds__(256) void k_lr_mm(LrMmArgs p) {
  __shared__ __attribute__((aligned(16))) float as[kMmStep][kMmTile];
  __shared__ __attribute__((aligned(16))) float bs[kMmStep][kMmTile];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int n0 = blockIdx.x * kMmTile, m0 = blockIdx.y * kMmTile;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < p.K; k0 += kMmStep) {
    __syncthreads();
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int e = tid + 256 * e4;  // 0 .. 1023: row e / 16, inner e % 16
      const int rr = e / kMmStep, kk = e % kMmStep;
      const int gk = k0 + kk;
      float va = 0.f, vb = 0.f;
      if (m0 + rr < p.M && gk < p.K) {
        const int64_t i = (int64_t)(m0 + rr) * p.K + gk;
        va = ABF16 ? bf2f(reinterpret_cast<const uint16_t *>(p.a)[i]) : reinterpret_cast<const float *>(p.a)[i];
      }
      if (n0 + rr < p.N && gk < p.K) vb = h2f(p.b[(int64_t)(n0 + rr) * p.K + gk]);
      as[kk][rr] = va;
      bs[kk][rr] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kMmStep; ++kk) {
      const float4 av = *reinterpret_cast<const float4 *>(&as[kk][4 * ty]);
      const float4 bv = *reinterpret_cast<const float4 *>(&bs[kk][4 * tx]);
      const float ar[4] = {av.x, av.y, av.z, av.w};
      const float br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * ty + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n >= p.N) continue;
      float *o = p.c + (int64_t)m * p.N + n;
      *o = ACC ? *o + acc[i][j] : acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_lowrank_tokens(const WView &w, const void *x, int xt, int batch, float *y, hipStream_t s) {
  if (w.lr_rank <= 0) return hipSuccess;
  LrTokArgs a{x, w.lr_u, w.lr_v, y, batch, w.k, w.lr_rank, w.n, 0};
  // Workgroups: enough rows each that the repeated t (r k B multiply-adds)
  // is at most about the rows' own r B per row times 4, and at most two per
  // compute unit.
  const int64_t per_wg_t = (int64_t)w.lr_rank * w.k;
  int64_t rows = per_wg_t / (4 * (int64_t)w.lr_rank);  // = k / 4
  rows = rows < 256 ? 256 : rows;
  int grid = (int)((w.n + rows - 1) / rows);
  const int cap = 2 * device_cu_count();
  grid = grid < 1 ? 1 : grid > cap ? cap : grid;
  a.rows_per_wg = (w.n + grid - 1) / grid;
  if (xt == VQ_BF16) launch_tokens_dt<true>(a, grid, s);
  else launch_tokens_dt<false>(a, grid, s);
  return hipGetLastError();
}

size_t lowrank_workspace_bytes(const WView &w, int m) {
  if (w.lr_rank <= 0 || m < 1) return 0;
  return (((size_t)m * w.lr_rank * 4) + 255) & ~(size_t)255;
}

hipError_t launch_lowrank_gemm(const WView &w, const uint16_t *x, int m, float *y, float *t, hipStream_t s) {
  if (w.lr_rank <= 0) return hipSuccess;
  const LrMmArgs pt{x, w.lr_v, t, m, w.lr_rank, w.k};
  hipLaunchKernelGGL((k_lr_mm<true, false>), dim3((unsigned)((w.lr_rank + kMmTile - 1) / kMmTile),
                                                   (unsigned)((m + kMmTile - 1) / kMmTile)),
                     dim3(256), 0, s, pt);
  const LrMmArgs py{t, w.lr_u, y, m, w.n, w.lr_rank};
  hipLaunchKernelGGL((k_lr_mm<false, true>), dim3((unsigned)((w.n + kMmTile - 1) / kMmTile),
                                                   (unsigned)((m + kMmTile - 1) / kMmTile)),
                     dim3(256), 0, s, py);
  return hipGetLastError();
}

}  // namespace vqmm
