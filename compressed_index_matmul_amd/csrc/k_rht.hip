// Randomized Hadamard transform of the input (GLQ page, "How it works":
// random sign flips, then a fast Walsh-Hadamard transform; "Bit widths":
// block-diagonal over power-of-two blocks).
//
// One workgroup per (token, block).  The block (<= 16384 fp32 = 64 KiB) lives
// in LDS; the first log2(R) butterfly stages (R = elements per thread) run in
// registers on a contiguous layout, the remaining stages run as radix-2
// passes through LDS.  Natural (Sylvester) order, orthonormal scaling applied
// once at the end.
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

// Blocks of nb = r * kRhtThreads elements (r = 8, 16 or 32, at most RM) with
// every block of every row 16-byte aligned in x, signs and out: each thread
// loads its r contiguous inputs and signs with vector loads, runs log2(r)
// stages in registers, and the remaining stages run two at a time (radix 4)
// through LDS.  r is uniform over the workgroup.
template <int RM, bool BF16>
__global__ __launch_bounds__(kRhtThreads) void k_rht_vec(RhtArgs a) {
  __shared__ float buf[kRhtMaxBlock];
  // element i lives at i ^ ((i >> 6) & 63): the six low bits are XORed with
  // the next six, so the register-stage stores (lane stride r = 8..32
  // floats) spread over all 64 banks, and 64-float runs stay conflict-free
  auto at = [](int i) { return i ^ ((i >> 6) & 63); };
  const int blk = blockIdx.x % a.nblocks;
  const int row = blockIdx.x / a.nblocks;
  int off, nb;
  rht_block(a, blk, off, nb);
  const int r = nb / kRhtThreads;  // 8, 16 or 32 (the launcher checks)
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)row * a.n + off;
  const int i0 = tid * r;
  float v[RM];
#pragma unroll
  for (int c = 0; c < RM / 8; ++c) {
    if (8 * c < r) {  // workgroup-uniform
      const uint2 su = *reinterpret_cast<const uint2 *>(a.signs + off + i0 + 8 * c);
      float xs[8];
      if (BF16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.x) + base + i0 + 8 * c);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xs[2 * e] = bf2f(w4[e] & 0xffffu);
          xs[2 * e + 1] = bf2f(w4[e] >> 16);
        }
      } else {
        const float4 *px = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + base + i0 + 8 * c);
        const float4 u0 = px[0], u1 = px[1];
        xs[0] = u0.x; xs[1] = u0.y; xs[2] = u0.z; xs[3] = u0.w;
        xs[4] = u1.x; xs[5] = u1.y; xs[6] = u1.z; xs[7] = u1.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * c + e] = xs[e] * (float)(int8_t)((e < 4 ? su.x : su.y) >> (8 * (e & 3)));
    }
  }
#pragma unroll
  for (int h = 1; h < RM; h <<= 1)
    if (h < r) {
#pragma unroll
      for (int q = 0; q < RM; ++q)
        if ((q & h) == 0 && q + h < RM) {
          const float p = v[q], m = v[q + h];
          v[q] = p + m;
          v[q + h] = p - m;
        }
    }
#pragma unroll
  for (int q = 0; q < RM; ++q)
    if (q < r) buf[at(i0 + q)] = v[q];
  // stages h = r, 2r, ...: two per pass on groups {i, i+h, i+2h, i+3h}.
  // A pass's r/4 groups per thread are disjoint, so all their loads go out
  // before any store (one LDS round trip per pass).
  int h = r, lh = __builtin_ctz((unsigned)r);
  for (; 4 * h <= nb; h *= 4, lh += 2) {
    __syncthreads();
    float x[RM];
    int ix[RM / 4];
#pragma unroll
    for (int it = 0; it < RM / 4; ++it)
      if (4 * it < r) {  // workgroup-uniform
        const int p = tid + it * kRhtThreads;
        const int i = ((p >> lh) << (lh + 2)) | (p & (h - 1));
        ix[it] = i;
        x[4 * it] = buf[at(i)];
        x[4 * it + 1] = buf[at(i + h)];
        x[4 * it + 2] = buf[at(i + 2 * h)];
        x[4 * it + 3] = buf[at(i + 3 * h)];
      }
#pragma unroll
    for (int it = 0; it < RM / 4; ++it)
      if (4 * it < r) {
        const int i = ix[it];
        const float x0 = x[4 * it], x1 = x[4 * it + 1], x2 = x[4 * it + 2], x3 = x[4 * it + 3];
        const float s0 = x0 + x1, d0 = x0 - x1, s1 = x2 + x3, d1 = x2 - x3;
        buf[at(i)] = s0 + s1;
        buf[at(i + h)] = d0 + d1;
        buf[at(i + 2 * h)] = s0 - s1;
        buf[at(i + 3 * h)] = d0 - d1;
      }
  }
  if (h < nb) {  // one stage left
    __syncthreads();
    float x[RM];
    int ix[RM / 2];
#pragma unroll
    for (int it = 0; it < RM / 2; ++it)
      if (2 * it < r) {
        const int p = tid + it * kRhtThreads;
        const int i = ((p >> lh) << (lh + 1)) | (p & (h - 1));
        ix[it] = i;
        x[2 * it] = buf[at(i)];
        x[2 * it + 1] = buf[at(i + h)];
      }
#pragma unroll
    for (int it = 0; it < RM / 2; ++it)
      if (2 * it < r) {
        buf[at(ix[it])] = x[2 * it] + x[2 * it + 1];
        buf[at(ix[it] + h)] = x[2 * it] - x[2 * it + 1];
      }
  }
  __syncthreads();
  const float sc = (float)(1.0 / __builtin_sqrt((double)nb));
  float4 *po = reinterpret_cast<float4 *>(a.out + base);
  for (int i = tid; i < nb / 4; i += kRhtThreads)
    po[i] = make_float4(buf[at(4 * i)] * sc, buf[at(4 * i + 1)] * sc, buf[at(4 * i + 2)] * sc, buf[at(4 * i + 3)] * sc);
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
  // vector path: every block is at least 8 * 512 elements long (so every
  // block offset is a multiple of 4096), and x, signs, out and the row pitch
  // keep 16-byte alignment
  const int xb = xt == VQ_F32 ? 4 : 2;
  const bool big_blocks = (a.nfull == 0 || max_block >= 8 * kRhtThreads) && a.rest % (8 * kRhtThreads) == 0;
  const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)signs % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
                       ((int64_t)n * xb % 16 == 0);
  if (big_blocks && aligned && r >= 8) {
    if (xt == VQ_BF16) {
      if (r <= 8) hipLaunchKernelGGL((k_rht_vec<8, true>), grid, dim3(kRhtThreads), 0, s, a);
      else if (r <= 16) hipLaunchKernelGGL((k_rht_vec<16, true>), grid, dim3(kRhtThreads), 0, s, a);
      else hipLaunchKernelGGL((k_rht_vec<32, true>), grid, dim3(kRhtThreads), 0, s, a);
    } else {
      if (r <= 8) hipLaunchKernelGGL((k_rht_vec<8, false>), grid, dim3(kRhtThreads), 0, s, a);
      else if (r <= 16) hipLaunchKernelGGL((k_rht_vec<16, false>), grid, dim3(kRhtThreads), 0, s, a);
      else hipLaunchKernelGGL((k_rht_vec<32, false>), grid, dim3(kRhtThreads), 0, s, a);
    }
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
