// Randomized Hadamard transform of the input (GLQ page, "How it works":
// random sign flips, then a fast Walsh-Hadamard transform; "Bit widths":
// block-diagonal over power-of-two blocks).
//
// One workgroup per (token, block).  The block (<= 16384 fp32 = 64 KiB) lives
// in LDS.  Blocks of at least 256 elements (k_rht_vec): the first four
// butterfly stages run in registers as the block is staged, the rest in
// passes of four (the last of up to five) through LDS.  Smaller blocks
// (k_rht): the first log2(R) stages in registers (R = elements per thread),
// the rest as radix-2 passes through LDS.  Natural (Sylvester) order,
// orthonormal scaling applied once.
#include "vqmm_device.h"
#include "vqmm_internal.h"

namespace vqmm {

constexpr int kRhtThreads = 512;
constexpr int kRhtMaxBlock = 16384;

struct RhtArgs {
  const void *x;
  const int8_t *signs;
  float *out;
  int n;          // row length
  int xt;         // VQ_F32 / VQ_BF16
  int nblocks;    // blocks per row
  int mb;         // max_block
  int nfull;      // n / max_block full blocks, then the set bits of the rest
  int rest;       // n % max_block
};

// Offset and length of block `b` of the greedy largest-first decomposition:
// nfull blocks of max_block, then one block per set bit of the remainder,
// largest first.
__device__ __forceinline__ void rht_block(const RhtArgs &a, int b, int &off, int &len) {
  if (b < a.nfull) {
    off = b * a.mb;
    len = a.mb;
    return;
  }
  off = a.nfull * a.mb;
  int j = b - a.nfull;
  for (int bit = 30; bit >= 0; --bit) {
    if (a.rest & (1 << bit)) {
      if (j == 0) {
        len = 1 << bit;
        return;
      }
      off += 1 << bit;
      --j;
    }
  }
  len = 0;  // unreachable for b < nblocks
}

// Blocks of at least 256 elements with every block of every row 16-byte
// aligned in x, signs and out.  A thread stages 16 consecutive elements
// times their signs and runs the first four butterfly stages on them in
// registers; the remaining stages run in passes of four through LDS (groups
// of 16 elements in registers, one barrier per pass), the last pass taking
// up to five and applying the orthonormal scale; then one coalesced store.
template <bool BF16>
__global__ __launch_bounds__(kRhtThreads) void k_rht_vec(RhtArgs a) {
  __shared__ __attribute__((aligned(16))) float buf[kRhtMaxBlock];
  const int blk = blockIdx.x % a.nblocks;
  const int row = blockIdx.x / a.nblocks;
  int off, nb;
  rht_block(a, blk, off, nb);
  int lb = 0;
  while ((1 << lb) < nb) ++lb;  // nb is a power of two >= 256
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)row * a.n + off;
  for (int g = tid; g < nb / 16; g += kRhtThreads) {
    float v[16];
    const void *xr = BF16 ? (const void *)(reinterpret_cast<const uint16_t *>(a.x) + base)
                          : (const void *)(reinterpret_cast<const float *>(a.x) + base);
    rht_load16(xr, !BF16, a.signs + off, 16 * g, v);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4 *>(&buf[16 * g + 4 * q]) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
  for (int s = 4; s < lb; s += (lb - s <= 5 ? 5 : 4)) {
    __syncthreads();
    fwht_pass<kRhtThreads>(buf, 0, 1, lb, s, 4, tid);
  }
  __syncthreads();
  float4 *po = reinterpret_cast<float4 *>(a.out + base);
  for (int i = tid; i < nb / 4; i += kRhtThreads) po[i] = reinterpret_cast<const float4 *>(buf)[i];
}

template <int R>
__global__ __launch_bounds__(kRhtThreads) void k_rht(RhtArgs a) {
  __shared__ float buf[kRhtMaxBlock];
  const int blk = blockIdx.x % a.nblocks;
  const int row = blockIdx.x / a.nblocks;
  int off, nb;
  rht_block(a, blk, off, nb);
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)row * a.n + off;
  // Contiguous layout: thread t owns elements R*t .. R*t+R-1 (when R*t < nb).
  const int r_eff = nb < R ? nb : R;  // blocks shorter than R use r_eff elements
  const int i0 = tid * r_eff;
  float v[R];
  if (i0 < nb) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (q < r_eff) {
        const int64_t gi = base + i0 + q;
        float xv = (a.xt == VQ_F32) ? reinterpret_cast<const float *>(a.x)[gi]
                                    : bf2f(reinterpret_cast<const uint16_t *>(a.x)[gi]);
        v[q] = xv * (float)a.signs[off + i0 + q];
      }
    }
    // in-register stages h = 1 .. r_eff/2
#pragma unroll
    for (int h = 1; h < R; h <<= 1) {
      if (h < r_eff) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
          if ((q & h) == 0 && q + h < r_eff) {
            const float p = v[q], m = v[q + h];
            v[q] = p + m;
            v[q + h] = p - m;
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < R; ++q)
      if (q < r_eff) buf[i0 + q] = v[q];
  }
  // remaining stages through LDS
  for (int h = r_eff; h < nb; h <<= 1) {
    __syncthreads();
    for (int p = tid; p < nb / 2; p += kRhtThreads) {
      const int i = (p / h) * 2 * h + (p % h);
      const float x0 = buf[i], x1 = buf[i + h];
      buf[i] = x0 + x1;
      buf[i + h] = x0 - x1;
    }
  }
  __syncthreads();
  const float sc = (float)(1.0 / __builtin_sqrt((double)nb));
  for (int i = tid; i < nb; i += kRhtThreads) a.out[base + i] = buf[i] * sc;
}

hipError_t launch_rht(const void *x, int xt, int batch, int n, const int8_t *signs, int max_block,
                      float *out, hipStream_t s) {
  RhtArgs a{};
  a.x = x;
  a.signs = signs;
  a.out = out;
  a.n = n;
  a.xt = xt;
  a.mb = max_block;
  a.nfull = n / max_block;
  a.rest = n % max_block;
  a.nblocks = a.nfull + __builtin_popcount((unsigned)a.rest);
  int maxlen = a.nfull ? max_block : 1;
  while (maxlen * 2 <= a.rest) maxlen *= 2;
  const dim3 grid((unsigned)((int64_t)batch * a.nblocks));
  // Elements per thread for the register stages: the largest block spread
  // over the workgroup (at least 1, at most 32 for a 16384 block).
  int r = maxlen / kRhtThreads;
  // vector path: every block is at least 256 elements long (so every block
  // offset is a multiple of 256), and x, signs, out and the row pitch keep
  // 16-byte alignment
  const int xb = xt == VQ_F32 ? 4 : 2;
  const bool big_blocks = (a.nfull == 0 || max_block >= 256) && a.rest % 256 == 0;
  const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)signs % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
                       ((int64_t)n * xb % 16 == 0);
  if (big_blocks && aligned) {
    if (xt == VQ_BF16) hipLaunchKernelGGL((k_rht_vec<true>), grid, dim3(kRhtThreads), 0, s, a);
    else hipLaunchKernelGGL((k_rht_vec<false>), grid, dim3(kRhtThreads), 0, s, a);
    return hipGetLastError();
  }
  if (r <= 1)
    hipLaunchKernelGGL(k_rht<1>, grid, dim3(kRhtThreads), 0, s, a);
  else if (r == 2)
    hipLaunchKernelGGL(k_rht<2>, grid, dim3(kRhtThreads), 0, s, a);
  else if (r == 4)
    hipLaunchKernelGGL(k_rht<4>, grid, dim3(kRhtThreads), 0, s, a);
  else if (r == 8)
    hipLaunchKernelGGL(k_rht<8>, grid, dim3(kRhtThreads), 0, s, a);
  else if (r == 16)
    hipLaunchKernelGGL(k_rht<16>, grid, dim3(kRhtThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_rht<32>, grid, dim3(kRhtThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace vqmm
