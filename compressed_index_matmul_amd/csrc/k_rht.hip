// Randomized Hadamard transform (GLQ page, "How it works": random sign
// flips, then a fast Walsh-Hadamard transform, its inverse inside the
// inference kernels; "Bit widths": block-diagonal over power-of-two blocks;
// "Inference kernels": the per-shard output transforms of a fused layer
// batched into one launch).
//
// Forward (the input side): signs, then the blocks' Hadamard.  Inverse (the
// output side): the blocks' Hadamard, then signs.  A row may be cut into up
// to kRhtMaxShards shards, each decomposed into blocks on its own; the grid
// is (token x block, shard).
//
// One workgroup per (token, block, shard).  The block (<= 16384 fp32 = 64
// KiB) lives in LDS.  Blocks of at least 256 elements (k_rht_vec): the first
// four butterfly stages run in registers as the block is staged, the rest in
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
  int n;        // row length (all shards)
  int xt;       // VQ_F32 / VQ_BF16
  int mb;       // max_block
  int nbx;      // grid.x per token: the most blocks of any shard
  int sh_off[kRhtMaxShards + 1];  // shard s is columns sh_off[s] .. sh_off[s + 1]
};

// Token, column offset and length of this workgroup's block (false: no
// block, the shard has fewer than nbx).  Within a shard of length L the
// greedy largest-first decomposition is L / mb blocks of mb, then one block
// per set bit of L % mb, largest first.
__device__ __forceinline__ bool rht_locate(const RhtArgs &a, int &row, int &off, int &len) {
  const int sh = blockIdx.y;
  const int s0 = a.sh_off[sh];
  const int slen = a.sh_off[sh + 1] - s0;
  const int nfull = slen / a.mb, rest = slen % a.mb;
  row = blockIdx.x / a.nbx;
  const int b = blockIdx.x % a.nbx;
  if (b >= nfull + __builtin_popcount((unsigned)rest)) return false;
  if (b < nfull) {
    off = s0 + b * a.mb;
    len = a.mb;
    return true;
  }
  off = s0 + nfull * a.mb;
  int j = b - nfull;
  for (int bit = 30; bit >= 0; --bit) {
    if (rest & (1 << bit)) {
      if (j == 0) {
        len = 1 << bit;
        return true;
      }
      off += 1 << bit;
      --j;
    }
  }
  return false;  // unreachable: b indexes a set bit
}

// Blocks of at least 256 elements with every block of every row 16-byte
// aligned in x, signs and out.  A thread stages 16 consecutive elements
// (times their signs when forward) and runs the first four butterfly stages
// on them in registers; the remaining stages run in passes of four through
// LDS (groups of 16 elements in registers, one barrier per pass), the last
// pass taking up to five and applying the orthonormal scale; then one
// coalesced store (times the signs when inverse).
template <bool BF16, bool INV>
__global__ __launch_bounds__(kRhtThreads) void k_rht_vec(RhtArgs a) {
  __shared__ __attribute__((aligned(16))) float buf[kRhtMaxBlock];
  int row, off, nb;
  if (!rht_locate(a, row, off, nb)) return;  // whole workgroup
  int lb = 0;
  while ((1 << lb) < nb) ++lb;  // nb is a power of two >= 256
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)row * a.n + off;
  for (int g = tid; g < nb / 16; g += kRhtThreads) {
    float v[16];
    const void *xr = BF16 ? (const void *)(reinterpret_cast<const uint16_t *>(a.x) + base)
                          : (const void *)(reinterpret_cast<const float *>(a.x) + base);
    rht_load16<!INV>(xr, !BF16, a.signs + off, 16 * g, v);
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
  for (int i = tid; i < nb / 4; i += kRhtThreads) {
    float4 v = reinterpret_cast<const float4 *>(buf)[i];
    if (INV) {
      const uint32_t sg = *reinterpret_cast<const uint32_t *>(a.signs + off + 4 * i);
      v.x *= (float)(int8_t)(sg & 0xffu);
      v.y *= (float)(int8_t)((sg >> 8) & 0xffu);
      v.z *= (float)(int8_t)((sg >> 16) & 0xffu);
      v.w *= (float)(int8_t)(sg >> 24);
    }
    po[i] = v;
  }
}

template <int R, bool INV>
__global__ __launch_bounds__(kRhtThreads) void k_rht(RhtArgs a) {
  __shared__ float buf[kRhtMaxBlock];
  int row, off, nb;
  if (!rht_locate(a, row, off, nb)) return;  // whole workgroup
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
        const float xv = (a.xt == VQ_F32) ? reinterpret_cast<const float *>(a.x)[gi]
                                          : bf2f(reinterpret_cast<const uint16_t *>(a.x)[gi]);
        v[q] = INV ? xv : xv * (float)a.signs[off + i0 + q];
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
  for (int i = tid; i < nb; i += kRhtThreads) {
    const float o = buf[i] * sc;
    a.out[base + i] = INV ? o * (float)a.signs[off + i] : o;
  }
}

template <bool INV>
static void launch_rht_dir(const RhtArgs &a, dim3 grid, bool vec, int xt, int r, hipStream_t s) {
  if (vec) {
    if (xt == VQ_BF16) hipLaunchKernelGGL((k_rht_vec<true, INV>), grid, dim3(kRhtThreads), 0, s, a);
    else hipLaunchKernelGGL((k_rht_vec<false, INV>), grid, dim3(kRhtThreads), 0, s, a);
  } else if (r <= 1) {
    hipLaunchKernelGGL((k_rht<1, INV>), grid, dim3(kRhtThreads), 0, s, a);
  } else if (r == 2) {
    hipLaunchKernelGGL((k_rht<2, INV>), grid, dim3(kRhtThreads), 0, s, a);
  } else if (r == 4) {
    hipLaunchKernelGGL((k_rht<4, INV>), grid, dim3(kRhtThreads), 0, s, a);
  } else if (r == 8) {
    hipLaunchKernelGGL((k_rht<8, INV>), grid, dim3(kRhtThreads), 0, s, a);
  } else if (r == 16) {
    hipLaunchKernelGGL((k_rht<16, INV>), grid, dim3(kRhtThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_rht<32, INV>), grid, dim3(kRhtThreads), 0, s, a);
  }
}

int rht_grid_blocks(int nsh, const int32_t *shard_len, int max_block) {
  int nbx = 0;
  for (int i = 0; i < nsh; ++i) {
    const int nb = shard_len[i] / max_block + __builtin_popcount((unsigned)(shard_len[i] % max_block));
    nbx = nb > nbx ? nb : nbx;
  }
  return nbx;
}

hipError_t launch_rht(const void *x, int xt, int batch, int n, int nsh, const int32_t *shard_len,
                      const int8_t *signs, int max_block, bool inverse, float *out, hipStream_t s) {
  RhtArgs a{};
  a.x = x;
  a.signs = signs;
  a.out = out;
  a.n = n;
  a.xt = xt;
  a.mb = max_block;
  a.nbx = rht_grid_blocks(nsh, shard_len, max_block);
  // vector path: every block of every shard is at least 256 elements long
  // (so every shard and block offset is a multiple of 256), and x, signs,
  // out and the row pitch keep 16-byte alignment
  bool big_blocks = true;
  int maxlen = 1;
  for (int i = 0; i < nsh; ++i) {
    a.sh_off[i + 1] = a.sh_off[i] + shard_len[i];
    const int nfull = shard_len[i] / max_block, rest = shard_len[i] % max_block;
    big_blocks = big_blocks && (nfull == 0 || max_block >= 256) && rest % 256 == 0;
    int ml = nfull ? max_block : 1;
    while (ml * 2 <= rest) ml *= 2;
    maxlen = ml > maxlen ? ml : maxlen;
  }
  const dim3 grid((unsigned)((int64_t)batch * a.nbx), (unsigned)nsh);
  // Elements per thread for the register stages: the largest block spread
  // over the workgroup (at least 1, at most 32 for a 16384 block).
  const int r = maxlen / kRhtThreads;
  const int xb = xt == VQ_F32 ? 4 : 2;
  const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)signs % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
                       ((int64_t)n * xb % 16 == 0);
  if (inverse) launch_rht_dir<true>(a, grid, big_blocks && aligned, xt, r, s);
  else launch_rht_dir<false>(a, grid, big_blocks && aligned, xt, r, s);
  return hipGetLastError();
}

}  // namespace vqmm
