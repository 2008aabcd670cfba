// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace vqmm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float h2f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// Exact double -> IEEE binary16 bits with one rounding to nearest, ties to
// even.  Subnormal results are kept, magnitudes that round past 65504 give
// infinity, the sign of zero is kept.  Integer arithmetic on the bit pattern,
// so there is no intermediate rounding.
__device__ __forceinline__ uint32_t f64_to_f16_rne(double d) {
  uint64_t b = (uint64_t)__double_as_longlong(d);
  uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  b &= 0x7fffffffffffffffull;
  if (b >= 0x7ff0000000000000ull) {  // inf or NaN
    return sign | 0x7c00u | (b > 0x7ff0000000000000ull ? 0x200u : 0u);
  }
  int e = (int)(b >> 52) - 1023;
  if (e < -25) return sign;  // |d| < 2^-25: rounds to zero
  if (e > 15) return sign | 0x7c00u;
  uint64_t m = (b & 0x000fffffffffffffull) | 0x0010000000000000ull;
  int E = e < -14 ? -14 : e;
  int shift = 42 + (E - e);  // keep units of 2^(E-10)
  uint64_t n = m >> shift;
  uint64_t rem = m & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (n & 1ull))) ++n;
  if (n == 2048) {
    n = 1024;
    ++E;
  }
  if (E > 15) return sign | 0x7c00u;
  if (n < 1024) return sign | (uint32_t)n;  // subnormal
  return sign | ((uint32_t)(E + 15) << 10) | (uint32_t)(n - 1024);
}

// The same rounding through the hardware conversions (a few instructions
// instead of some forty), for finite |d| < 65504: d is rounded to float with
// the low bit forced to 1 when inexact (round to odd: the float has 24
// significant bits, at least two more than binary16's 11, so the float ->
// binary16 rounding to nearest even then equals the direct one).
__device__ __forceinline__ uint32_t f64_to_f16_rn_odd(double d) {
  const float f = (float)d;  // nearest, ties to even
  uint32_t fb = __float_as_uint(f);
  const double back = (double)f;
  if (back != d) {
    if (__builtin_fabs(back) > __builtin_fabs(d)) fb -= 1u;  // the float toward zero
    fb |= 1u;                                                  // sticky bit
  }
  const _Float16 h = (_Float16)__uint_as_float(fb);          // nearest, ties to even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Sum over the 64 lanes of a wave in a fixed order (DPP within rows of 16,
// then the four row totals added lane 0 + 16 + 32 + 48).  Result valid in
// every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)); // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true)); // row_mirror
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// 16-byte global -> LDS direct load (global_load_lds_dwordx4): lane l writes
// its 16 bytes at lds_wave_base + 16 l.  `lds_wave_base` must be the same
// for the whole wave.  The builtin exists only for the GPU target, so the
// host compilation pass (which never runs device code) sees an empty body.
__device__ __forceinline__ void lds_direct_16(const void *src, void *lds_wave_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
#else
  (void)src;
  (void)lds_wave_base;
#endif
}

// A wave-uniform pointer as a value held in scalar registers.  Selecting
// between such values cannot be folded back into a load from a computed
// address in the kernel-argument block (which, with a per-lane selector,
// becomes a vector load and a wait).
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

// Scheduling fence: the compiler may not move instructions across it (keeps
// prefetch loads where they are issued instead of sinking them to their use).
__device__ __forceinline__ void sched_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// Scheduling-group hint: the next `n` instructions of the region that match
// `mask` (0x002 VALU, 0x008 MFMA, 0x100 LDS read, 0x200 LDS write, 0x020
// global read) form one group, groups in program order of these calls.
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
#endif
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order).  gfx9 s_waitcnt immediate: vmcnt bits
// [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]; the other two counters
// are left at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt holds 0..63");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}

// Workgroup barrier for data in LDS: waits for this wave's LDS operations
// (lgkmcnt 0), then meets the other waves; the memory clobber keeps the
// compiler from moving memory accesses across it.  Unlike __syncthreads()
// it does not wait for outstanding vector-memory loads (whose fence, with an
// LDS-direct copy in flight, becomes a wait for every load of the wave): the
// caller first waits (wait_vmem) for the LDS-direct copies that must have
// landed, and loads issued after them, e.g. index rows from HBM, stay in
// flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
}

// Wait for every outstanding memory operation of the wave.
__device__ __forceinline__ void wait_all_memory() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0);
#endif
}

// Raw buffer resources (CDNA buffer descriptors): a loaded element is the
// base address plus a 32-bit per-lane offset plus a wave-uniform offset kept
// in a scalar register, so a load needs no per-lane 64-bit address math.
// The builtins exist only for the GPU target; the host pass sees stubs.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buf_t;
#else
typedef const void *buf_t;
#endif
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Descriptor for `bytes` bytes at p (raw, no stride; dword 3 = 0x00020000,
// the plain 32-bit data format used for raw buffers on gfx9).
__device__ __forceinline__ buf_t make_buf(const void *p, uint32_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
#else
  (void)bytes;
  return p;
#endif
}
__device__ __forceinline__ uint32_t buf_u8(buf_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
#else
  (void)r, (void)voff, (void)soff;
  return 0;
#endif
}
__device__ __forceinline__ uint32_t buf_u16(buf_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
#else
  (void)r, (void)voff, (void)soff;
  return 0;
#endif
}
__device__ __forceinline__ uint32_t buf_u32(buf_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
#else
  (void)r, (void)voff, (void)soff;
  return 0;
#endif
}
__device__ __forceinline__ uint2 buf_u64(buf_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v.x, v.y);
#else
  (void)r, (void)voff, (void)soff;
  return make_uint2(0, 0);
#endif
}
__device__ __forceinline__ uint4 buf_u128(buf_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  (void)r, (void)voff, (void)soff;
  return make_uint4(0, 0, 0, 0);
#endif
}

// Store one float at descriptor + lane offset + wave-uniform offset (a
// vector-memory store).  The hardware range check of raw buffers does not
// include the scalar offset, so callers keep every store inside the buffer
// themselves.
__device__ __forceinline__ void buf_store_f32(float v, buf_t r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
#else
  (void)v, (void)r, (void)voff, (void)soff;
#endif
}

// Index of flat group f of stage planes (any width: 16-bit words; 12-bit
// low byte plus nibble; 8-bit byte; 4-bit nibble).
__device__ __forceinline__ uint32_t load_index(int bits, const uint8_t *lo, const uint8_t *hi,
                                               const uint16_t *i16, size_t f) {
  if (bits == 16) return i16[f];
  const uint32_t nib = bits == 8 ? 0u : ((uint32_t)(hi[f >> 1] >> ((f & 1) * 4)) & 0xfu);
  if (bits == 4) return nib;
  uint32_t v = lo[f];
  if (bits == 12) v |= nib << 8;
  return v;
}

// Index widths of the residual stages fixed at compile time (0 = no such
// stage), for the kernels that keep every codebook in LDS.  A 12-bit index
// is a low-byte plane plus a nibble plane shifted up by 8, an 8-bit index the
// byte plane alone, a 4-bit index the nibble plane alone.  The stages'
// codebooks sit back to back in LDS, stage t from row off(t).
__host__ __device__ constexpr int ladder_rows(int b) { return b > 0 ? 1 << b : 0; }
__host__ __device__ constexpr int ladder_planes(int b) { return b == 12 ? 2 : b > 0 ? 1 : 0; }

template <int B0, int B1 = 0, int B2 = 0, int B3 = 0>
struct Ladder {
  static_assert((B0 == 4 || B0 == 8 || B0 == 12) && (B1 == 0 || B1 == 4 || B1 == 8 || B1 == 12) &&
                    (B2 == 0 || B2 == 4 || B2 == 8 || B2 == 12) && (B3 == 0 || B3 == 4 || B3 == 8 || B3 == 12),
                "LDS ladders take 4-, 8- and 12-bit stages");
  static_assert((B1 > 0 || B2 == 0) && (B2 > 0 || B3 == 0), "stages are consecutive");
  static constexpr int S = 1 + (B1 > 0) + (B2 > 0) + (B3 > 0);
  static constexpr int kRows = ladder_rows(B0) + ladder_rows(B1) + ladder_rows(B2) + ladder_rows(B3);
  // index loads per group chunk (one per plane)
  static constexpr int kPlanes = ladder_planes(B0) + ladder_planes(B1) + ladder_planes(B2) + ladder_planes(B3);
  // every stage has the same width
  static constexpr bool kUniform = (B1 == 0 || B1 == B0) && (B2 == 0 || B2 == B0) && (B3 == 0 || B3 == B0);
  // every stage's codebook is whole 64-row (1 KiB) blocks
  static constexpr bool kBlocks = B0 >= 8 && (B1 == 0 || B1 >= 8) && (B2 == 0 || B2 >= 8) && (B3 == 0 || B3 >= 8);
  __host__ __device__ static constexpr int bits(int t) { return t == 0 ? B0 : t == 1 ? B1 : t == 2 ? B2 : t == 3 ? B3 : 0; }
  __host__ __device__ static constexpr int off(int t) {
    return (t > 0 ? ladder_rows(B0) : 0) + (t > 1 ? ladder_rows(B1) : 0) + (t > 2 ? ladder_rows(B2) : 0);
  }
  __host__ __device__ static constexpr bool lo(int t) { return bits(t) == 8 || bits(t) == 12; }
  __host__ __device__ static constexpr bool hi(int t) { return bits(t) == 4 || bits(t) == 12; }
  __host__ __device__ static constexpr int hshift(int t) { return bits(t) == 12 ? 8 : 0; }
  // stage owning codebook row `row` of the back-to-back layout
  __host__ __device__ static constexpr int stage_of(int row) {
    return (S > 1 && row >= off(1)) + (S > 2 && row >= off(2)) + (S > 3 && row >= off(3));
  }
};

// Copy the codebooks of a mixed-width ladder LD into LDS, back to back (stage
// t from row LD::off(t)), with LDS-direct loads: NW waves, 64 rows (1 KiB)
// per wave and load.  A block inside one stage is one load from a
// wave-uniform stage; a block that spans stages or ends early (16-row 4-bit
// codebooks) is copied row by row, lanes past the last row masked off.  The
// stage pointers are selected among values held in scalar registers (an
// index into the argument array would become a vector load and a wait
// before every block).  The caller waits for the loads and synchronises.
template <class LD, int NW>
__device__ __forceinline__ void stage_ladder_lds(const uint16_t *const *cb, uint4 *s_cb, int wave, int lane) {
  constexpr int S = LD::S;
  constexpr int CBN = LD::kRows;
  const uint4 *cb0 = static_cast<const uint4 *>(uniform_ptr(cb[0]));
  const uint4 *cb1 = static_cast<const uint4 *>(uniform_ptr(S > 1 ? cb[1] : cb[0]));
  const uint4 *cb2 = static_cast<const uint4 *>(uniform_ptr(S > 2 ? cb[2] : cb[0]));
  const uint4 *cb3 = static_cast<const uint4 *>(uniform_ptr(S > 3 ? cb[3] : cb[0]));
  auto cbp = [&](int t) { return t == 0 ? cb0 : t == 1 ? cb1 : t == 2 ? cb2 : cb3; };
#pragma unroll
  for (int r = 0; r < (CBN + NW * 64 - 1) / (NW * 64); ++r) {
    const int blk = (r * NW + wave) * 64;  // wave-uniform
    if (blk < CBN) {
      const int t0 = LD::stage_of(blk);
      if (blk + 64 <= LD::off(t0) + ladder_rows(LD::bits(t0))) {
        lds_direct_16(cbp(t0) + (blk - LD::off(t0)) + lane, s_cb + blk);
      } else {
        const int row = blk + lane;
        if (row < CBN) {
          const int t = LD::stage_of(row);
          lds_direct_16(cbp(t) + (row - LD::off(t)), s_cb + blk);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fast Walsh-Hadamard transform pieces (GLQ page, "How it works": random
// sign flips, then a fast Walsh-Hadamard transform; "Bit widths": blocks of
// powers of two), shared by rht_apply and the 16-bit decode kernel.
// ---------------------------------------------------------------------------

// Elements i .. i + 15 of x (fp32 or bf16, 16-byte aligned) times their
// signs (int8, 16-byte aligned; not read without SIGNS), then butterfly
// stages 1, 2, 4, 8 (the low four bits of the index) in registers,
// Sylvester order.
template <bool SIGNS = true>
__device__ __forceinline__ void rht_load16(const void *x, bool f32, const int8_t *signs, size_t i, float (&v)[16]) {
  if (f32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 t = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(x) + i + 4 * q);
      v[4 * q] = t.x, v[4 * q + 1] = t.y, v[4 * q + 2] = t.z, v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(x) + i + 8 * q);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * q + 2 * e] = bf2f(w4[e] & 0xffffu);
        v[8 * q + 2 * e + 1] = bf2f(w4[e] >> 16);
      }
    }
  }
  if (SIGNS) {
    const uint4 sg = *reinterpret_cast<const uint4 *>(signs + i);
    const uint32_t s4[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= (float)(int8_t)((s4[j >> 2] >> (8 * (j & 3))) & 0xffu);
  }
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((j & h) == 0) {
        const float p0 = v[j], p1 = v[j + h];
        v[j] = p0 + p1;
        v[j + h] = p0 - p1;
      }
}

// One group of a FWHT pass: the R elements base + j 2^s (j < R) of s_x,
// R = 2^r butterfly stages in registers; the result times sc.  With s == 0
// the elements are contiguous and move as 16-byte LDS accesses.
template <int R>
__device__ __forceinline__ void fwht_group(float *s_x, int base, int s, float sc) {
  float v[R];
  if (R >= 4 && s == 0) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const float4 t = *reinterpret_cast<const float4 *>(&s_x[base + 4 * q]);
      v[4 * q] = t.x, v[4 * q + 1] = t.y, v[4 * q + 2] = t.z, v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = s_x[base + (j << s)];
  }
#pragma unroll
  for (int h = 1; h < R; h <<= 1)
#pragma unroll
    for (int j = 0; j < R; ++j)
      if ((j & h) == 0) {
        const float p0 = v[j], p1 = v[j + h];
        v[j] = p0 + p1;
        v[j + h] = p0 - p1;
      }
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] *= sc;
  if (R >= 4 && s == 0) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q)
      *reinterpret_cast<float4 *>(&s_x[base + 4 * q]) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else {
#pragma unroll
    for (int j = 0; j < R; ++j) s_x[base + (j << s)] = v[j];
  }
}

// Pass s over `count` blocks of 2^lb elements from offset off (bits [s, s +
// r) of the in-block index: r = 4, or all that is left when that is at most
// 5, so no pass of a single stage remains): the groups of all these
// blocks spread over the NT threads; a block whose last bits these are is
// scaled by 1/sqrt(2^lb).
template <int NT>
__device__ __forceinline__ void fwht_pass(float *s_x, int off, int count, int lb, int s, int s0, int tid) {
  // passes start at s0, s0 + 4, ...; a block is done once a pass took its
  // last bits (at most 5 of them), so later passes skip it
  if (s >= lb || count <= 0 || (s > s0 && lb - (s - 4) <= 5)) return;
  const int r = lb - s <= 5 ? lb - s : 4;
  const bool last = s + r >= lb;
  const float sc = last ? (float)(1.0 / __builtin_sqrt((double)(1 << lb))) : 1.f;
  const int gpb_log = lb - r;  // log2 groups per block
  const int groups = count << gpb_log;
  for (int gid = tid; gid < groups; gid += NT) {
    const int blk = gid >> gpb_log;
    const int gi = gid & ((1 << gpb_log) - 1);
    const int base = off + (blk << lb) + ((gi >> s) << (s + r)) + (gi & ((1 << s) - 1));
    switch (r) {
      case 5: fwht_group<32>(s_x, base, s, sc); break;
      case 4: fwht_group<16>(s_x, base, s, sc); break;
      case 3: fwht_group<8>(s_x, base, s, sc); break;
      case 2: fwht_group<4>(s_x, base, s, sc); break;
      default: fwht_group<2>(s_x, base, s, sc); break;
    }
  }
}

// The input transform: signs (null: none) and the largest block.
struct RhtIn {
  const int8_t *signs;
  int mb;
};

// In-place orthonormal FWHT of every block of s_x[0, K): K / mb blocks of
// mb, then one block per set bit of K % mb, largest first.  Passes of up to
// four stages, one barrier each; the blocks of mb are one flat loop over
// their groups, the few remainder blocks one loop each.
// s0: the first in-block bit left to transform (4 when the staging has done
// bits 0..3).
template <int NT>
__device__ __forceinline__ void fwht_lds(float *s_x, int K, int mb, int tid, int s0) {
  const int nfull = K / mb, rest = K % mb;
  int maxbits = 0;
  for (int p = mb; p > 1; p >>= 1) ++maxbits;
  // passes at s0, s0 + 4, ...: a block's last pass takes its remaining 1..5
  // bits (the loop stops at maxbits - 1 so a 5-bit remainder is one pass)
  for (int s = s0; s < maxbits; s += (maxbits - s <= 5 ? 5 : 4)) {
    __syncthreads();  // the previous pass (or the staging) is complete
    fwht_pass<NT>(s_x, 0, nfull, maxbits, s, s0, tid);
    int off = nfull * mb;
    for (int bit = maxbits - 1; bit >= 0; --bit)  // uniform
      if (rest & (1 << bit)) {
        fwht_pass<NT>(s_x, off, 1, bit, s, s0, tid);
        off += 1 << bit;
      }
  }
}

}  // namespace vqmm
