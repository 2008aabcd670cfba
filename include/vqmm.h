/*
 * vqmm.h -- C ABI of libvqmm, the MI355X (gfx950) compressed-index matmul.
 *
 * A linear layer's weight W [n_out, k_in] (nn.Linear layout) is stored as
 * vector-quantization codebook indices: every group of 8 consecutive
 * input-dim weights of a row is one index per residual stage into that
 * stage's per-tensor codebook of 8-wide fp16 vectors, and a group decodes to
 *
 *     w[r, 8g + j] = s[r, (8g) / scale_block] * sum_t codebook_t[idx_t[r, g]][j]
 *
 * (orka README, "How it works": groups of 8 weights, per-tensor codebooks,
 * indices stored as 12-bit bit-planes, decode = scale times the sum of the
 * indexed codebook entries; GLQ page, "How it works" / "Bit widths": 16-bit
 * indices into a 65,536-entry codebook, residual stages).  The products below
 * take Y = X dequant(W)^T without writing the dense W to memory (GLQ page,
 * "Inference kernels").
 *
 * Conventions for every entry point:
 *  - All array pointers are device pointers owned by the caller; the library
 *    never frees them and keeps no reference after the call returns.  Base
 *    pointers must be 16-byte aligned (VQ_ERR_ALIGN otherwise).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously on it; the call returns before it finishes.
 *    Inputs and outputs must not alias.
 *  - Every argument is validated on the host before any HIP call, so invalid
 *    arguments return an error with nothing enqueued and no device touched.
 *    A failed launch returns VQ_ERR_HIP.  No C++ exception crosses the ABI.
 *  - The library allocates no device memory and holds no per-call state;
 *    calls on different streams may run concurrently.  Scratch memory, where
 *    a kernel needs any, is the caller's workspace (vq_gemm), except for
 *    vq_gemm_noalloc, which uses a static device array of the library and
 *    must not overlap with another vq_gemm_noalloc call on the same GPU.
 *  - Results are deterministic: fixed reduction order, no atomics.
 */
#ifndef VQMM_H
#define VQMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQMM_VERSION 5
#define VQ_MAX_STAGES 4

/* vq_weight.flags: stage_scale[] holds one residual scale per stage. */
#define VQ_STAGE_SCALES 1
/* Largest rank of a low-rank correction (vq_weight.lr_rank). */
#define VQ_MAX_LR_RANK 256

/* Status codes returned by every entry point. */
typedef enum vq_status {
  VQ_OK = 0,
  VQ_ERR_NULL = -1,        /* a required pointer is NULL */
  VQ_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  VQ_ERR_DTYPE = -3,       /* unsupported element type for this argument */
  VQ_ERR_UNSUPPORTED = -4, /* valid request outside what the kernels implement */
  VQ_ERR_ALIGN = -5,       /* a base pointer is not 16-byte aligned */
  VQ_ERR_HIP = -6,         /* the HIP runtime reported an error */
  VQ_ERR_VALUE = -7,       /* a scalar argument value is invalid (a non-finite stage scale) */
  VQ_ERR_WORKSPACE = -8    /* the caller's workspace is smaller than vq_gemm_workspace_size */
} vq_status;

/* Element types of activations. */
typedef enum vq_dtype { VQ_F32 = 0, VQ_BF16 = 1 } vq_dtype;

/*
 * Descriptor of one compressed weight (array pointers are device memory).
 *
 * Groups are numbered row-major: group g of output row r is f = r*(k_in/8)+g.
 * Stage t < n_stages has index width b_t = stage_bits[t] when that is
 * non-zero, else idx_bits.  By width:
 *   16 : idx16[t]   uint16 [n_out*k_in/8]        little-endian index
 *        (GLQ page, "How it works": one 16-bit index per 8 weights)
 *   12 : idx_lo[t]  uint8  [n_out*k_in/8]        bits 0..7 of index f
 *        idx_hi[t]  uint8  [ceil(n_out*k_in/16)] bits 8..11: low nibble of
 *                   idx_hi[t][f/2] for even f, high nibble for odd f
 *        (orka README, "How it works": 12-bit bit-planes, a low byte plus
 *        packed high bits; the nibble order is this library's reading)
 *   8  : idx_lo[t]  uint8  [n_out*k_in/8]        index = idx_lo[t][f]
 *   4  : idx_hi[t]  uint8  [ceil(n_out*k_in/16)] index = the nibble of f,
 *                   packed as the 12-bit high plane (the residual stage of
 *                   orka's rvq-12-4 mode: 12 + 4 bits per 8 weights)
 * Mixed widths form the residual ladders of the GLQ page, "Bit widths" (a
 * 16-bit primary plus 8- or 16-bit residual stages, up to four stages).
 * codebook[t] : fp16 bits [2^b_t][8], row-major.
 * scales      : fp16 bits [n_out][ceil(k_in/scale_block)]; column c of row r
 *               uses scales[r][c / scale_block].  scale_block >= k_in means
 *               one scale per row.
 * flags       : 0, or VQ_STAGE_SCALES: stage t's codebook entries are
 *               multiplied by the float stage_scale[t] (finite), the residual
 *               scale of the GLQ page's two-stage call ("Inference kernels"):
 *                 w[r, 8g + j] = s[r, blk] * sum_t stage_scale[t] * cb_t[..][j].
 *               Without the flag every stage scale is 1.
 * sp_*        : optional sparse correction added to the decoded weight (orka
 *               README, "How it works": the decode plus a sparse correction;
 *               its correct command adds one), CSR over output rows:
 *                 w[r, sp_col[j]] += fp16 sp_val[j],  sp_rowptr[r] <= j < sp_rowptr[r+1],
 *               added after the block scale, unscaled, entries of a row in
 *               storage order (repeated columns sum).  Device data the caller
 *               keeps consistent: sp_rowptr[0] = 0, non-decreasing,
 *               sp_rowptr[n_out] = sp_nnz; columns ascending within a row and
 *               < k_in.  Kernels clamp row ranges to [0, sp_nnz] and skip
 *               columns >= k_in, so inconsistent data gives wrong values,
 *               never an access outside these arrays.
 * lr_*        : optional low-rank correction added to the decoded weight
 *               (orka README, CLI: the correct command adds a low-rank or
 *               sparse correction; the pages give no form, this is the
 *               library's reading): fp16 factors U = lr_u [n_out][lr_rank]
 *               and V = lr_v [lr_rank][k_in], both row-major,
 *                 w[r, c] += sum_j U[r][j] V[j][c],
 *               after the sparse entries.  The products never form U V:
 *               they compute t = x V^T, then y += t U^T, in fp32 with a
 *               fixed order, so the error of this term is bounded relative
 *               to sum_j |U[r][j]| sum_c |V[j][c] x[c]| (see vq_gemv).
 * Unused pointer slots and unused stage_bits / stage_scale entries are
 * ignored.  A zero-initialised descriptor with the first block filled in
 * describes a uniform ladder without stage scales or correction.
 */
typedef struct vq_weight {
  int32_t n_out;       /* N >= 1 */
  int32_t k_in;        /* K >= 8, K % 8 == 0; n_out*k_in < 2^31 */
  int32_t n_stages;    /* 1..4 */
  int32_t idx_bits;    /* 4, 8, 12 or 16: width of every stage without its own */
  int32_t scale_block; /* columns per scale, >= 8 and a multiple of 8 */
  int32_t flags;       /* 0 or VQ_STAGE_SCALES */
  const uint8_t *idx_lo[VQ_MAX_STAGES];
  const uint8_t *idx_hi[VQ_MAX_STAGES];
  const uint16_t *idx16[VQ_MAX_STAGES];
  const uint16_t *codebook[VQ_MAX_STAGES];
  const uint16_t *scales;
  int32_t stage_bits[VQ_MAX_STAGES]; /* 0 (= idx_bits), 4, 8, 12 or 16 */
  float stage_scale[VQ_MAX_STAGES];  /* used with VQ_STAGE_SCALES */
  int32_t sp_nnz;                    /* entries of the sparse correction, 0 = none */
  int32_t sp_reserved;               /* set to 0 */
  const int32_t *sp_rowptr;          /* [n_out + 1] (when sp_nnz > 0) */
  const int32_t *sp_col;             /* [sp_nnz] */
  const uint16_t *sp_val;            /* fp16 bits [sp_nnz] */
  int32_t lr_rank;                   /* rank of the low-rank correction, 0 = none, 1..VQ_MAX_LR_RANK */
  int32_t lr_reserved;               /* set to 0 */
  const uint16_t *lr_u;              /* fp16 bits [n_out][lr_rank] (when lr_rank > 0) */
  const uint16_t *lr_v;              /* fp16 bits [lr_rank][k_in] */
} vq_weight;

/* Library version (VQMM_VERSION).  Host only. */
int vq_version(void);

/* Static text for a status code.  Host only. */
const char *vq_status_string(int status);

/* Validate a descriptor without touching the device.  Returns VQ_OK or the
 * error the compute entry points would return for it.  Host only. */
int vq_validate(const vq_weight *w);

/* Stored bytes of the weight: index planes + fp16 scales + fp16 codebooks,
 * each counted once (per group and stage: 16-bit 2 bytes, 12-bit 1.5, 8-bit
 * 1, 4-bit 0.5, nibble planes rounded up), plus a sparse correction's
 * 4 (n_out + 1) + 6 sp_nnz bytes and a low-rank correction's 2 lr_rank
 * (n_out + k_in) bytes.  Negative vq_status on an invalid descriptor.  Host
 * only. */
int64_t vq_compressed_bytes(const vq_weight *w);

/*
 * Unpack and/or dequantize the whole weight (orka README, "How it works":
 * bit-plane storage and the scale-times-sum decode).  Not on the matmul path;
 * it exists to check the format and for callers that want the dense weight.
 *   idx_out : uint16 [n_stages][n_out][k_in/8] unpacked indices, or NULL
 *   w_out   : fp16 bits [n_out][k_in], or NULL.  Each weight is the exact
 *             value of the decode formula rounded once to fp16 (nearest,
 *             ties to even; subnormals kept, overflow to +-inf).  With
 *             VQ_STAGE_SCALES the value is not exact in general and is
 *             defined by a fixed float64 order: each stage_scale[t] * entry
 *             (exact), summed from stage 0 up with float64 rounding, times
 *             the block scale in float64, then rounded once to fp16.  A
 *             sparse correction is added to that float64 value, entry by
 *             entry in storage order, then a low-rank correction's terms
 *             U[r][j] V[j][c] (exact products) for j = 0, 1, ... in order,
 *             each addition rounded to float64, before the one rounding.
 * At least one output must be non-NULL.  Bit-exact.
 */
int vq_unpack_dequant(const vq_weight *w, uint16_t *idx_out, uint16_t *w_out, void *stream);

/*
 * Decode-style product y = x dequant(W)^T for 1..16 tokens (GLQ page,
 * "Inference kernels": each output row walks its k_in/8 groups, gathering
 * codebook vectors; B = 1 is a matrix-vector product).
 *   x     : [batch][k_in], VQ_F32 (float) or VQ_BF16 (bf16 bits)
 *   batch : 1..16
 *   y     : float [batch][n_out]
 * One token, or fp32 tokens: exact fp16 codebook products accumulated in fp32
 * (bf16 x is held in fp16 after a power-of-two rescale per 32 columns, exact
 * for every value within 2^28 of the largest |x| of its 32), so every output
 * satisfies |y - y_exact| <= 2e-3 * sum_k |w x| + 1e-6.  One exception: on
 * a single 16-bit stage with one scale per row and n_out * k_in >= 2^25
 * (the codebook-sliced kernel), fp32 x is held in fp16 after a power-of-two
 * rescale per 16 U columns, i.e. rounded to 11 significant bits, so the
 * bound there is (2^-11 + k_in 2^-24) sum_k |w x| + 1e-6 (inside 2e-3 for
 * k_in <= 16384); bf16 x stays exact on that kernel.
 * 2..4 bf16 tokens whose rows are short enough (k_in <= 6144, and the
 * codebooks plus every token's x fit on chip) use the same exact fp16
 * products, one launch for all tokens.  Other 2..16 bf16 tokens run on bf16
 * matrix cores as vq_gemm does with 16 tokens or fewer: each decoded weight
 * w enters as two bf16 parts, hi = bf16(w) and lo = bf16(w - hi) (|w - hi -
 * lo| <= 2^-17 |w|), multiplied in two MFMAs with exact products and fp32
 * sums of 2 k_in terms, so every output satisfies |y - y_exact| <= (2^-17 +
 * 2^-20 + 2 k_in 2^-24) sum_k |w x| + 1e-6, inside 2e-3 * sum_k |w x| + 1e-6
 * for any x when k_in <= 16384.  A sparse
 * correction adds x S^T (fp16 values times x, fp32 sums) in a second launch
 * on the same stream.  A low-rank correction adds (x V^T) U^T in one more
 * launch with no scratch: every workgroup forms t = x V^T for all tokens
 * itself (fp32, fixed order), then adds t U^T to its rows of y; its term
 * is within 2e-3 * sum_j |U[r][j]| sum_c |V[j][c] x[c]| (k_in <= 16384).
 */
int vq_gemv(const vq_weight *w, const void *x, int32_t x_dtype, int32_t batch, float *y,
            void *stream);

/*
 * Many-token product y = x dequant(W)^T (GLQ page, "Inference kernels":
 * tensor-core path for batched inputs).  Decoded weight tiles are rounded on
 * chip to a 16-bit type and multiplied on matrix cores with fp32
 * accumulation.  Two paths:
 *  - fp16 (more than 64 tokens, k_in % 256 == 0, scale_block % 32 == 0,
 *    m rounded up to 16 times k_in below 2^31, one stage of 8 or 12 bits
 *    or two stages 12+12, 12+4, 8+8, 8+4): x is first
 *    converted into the workspace to fp16 after a power-of-two rescale per
 *    token (exact for every value within 2^28 of the token's largest |x|,
 *    smaller ones off by at most 2^-39 of it), each weight is rounded to
 *    fp16 (relative error <= 2^-10 + 2^-22), and the bound is |y - y_exact|
 *    <= (2^-10 + 2^-22 + k_in 2^-24) sum_k |w x| + 1e-6, inside
 *    2e-3 * sum_k |w x| + 1e-6 for any x when k_in <= 16384;
 *  - bf16 (every other call, including all calls with 64 tokens or fewer):
 *    see the bound below.  With 16 tokens or fewer, and with 17..64 tokens
 *    on the few-token unit kernel (stages of 8 bits, up to four, or of 12
 *    bits, up to two, or the ladders 12+4 and 8+4; k_in % 256 == 0,
 *    scale_block % 128 == 0, n_out up to 128 times the CU count, i.e.
 *    32768 rows on 256 CUs), the weights enter as bf16 hi + lo parts
 *    and the bound is vq_gemv's (inside 2e-3 * sum_k |w x| + 1e-6 for any x
 *    when k_in <= 16384).
 *   x         : bf16 bits [m][k_in];  m >= 1, m * k_in and m * n_out below
 *               2^31 (VQ_ERR_SHAPE otherwise); with a low-rank correction
 *               at most 65535 * 64 tokens (VQ_ERR_UNSUPPORTED otherwise)
 *   y         : float [m][n_out]
 *   workspace : device scratch of ws_bytes bytes owned by the caller, 16-byte
 *               aligned, or NULL when ws_bytes == 0.  It must hold at least
 *               vq_gemm_workspace_size(w, m) bytes (VQ_ERR_WORKSPACE
 *               otherwise, before any HIP call); its contents on entry are
 *               ignored and on return unspecified.  Kernels of the same call
 *               use it in stream order; two calls in flight at the same time
 *               need two workspaces.  (The GLQ page, "Inference kernels",
 *               keeps split-K partials in such a scratch buffer for a fixed
 *               reduction order; here split-K sums meet in LDS in a fixed
 *               order, and the workspace holds the fp16 x and a low-rank
 *               correction's t.)
 * On the bf16 path x is used as given and the workspace holds only a
 * low-rank correction's t.  Where the weights do not enter as hi + lo
 * parts (more than 16 tokens off the few-token unit kernel), bf16 keeps 8
 * significant bits, so each weight carries a relative error of up to 2^-8:
 * the guaranteed bound is |y - y_exact| <= (2^-8 + 2^-23 + k_in 2^-24)
 * sum_k |w x| + 1e-6.  For dense activations the rounding errors average
 * out and outputs stay well inside 2e-3 * sum_k |w x| + 1e-6 (about 0.07
 * of it at k_in = 4096 for N(0,1) inputs); a one-hot or very short x can
 * exceed that tighter bound.  A sparse correction adds x S^T exactly as
 * vq_gemv does (fp32, not rounded to bf16).  A low-rank correction takes
 * two more launches: t = x V^T into the workspace (m * lr_rank floats after
 * the fp16 path's part, 256-byte aligned), then y += t U^T, both fp32 with
 * a fixed order, within the same bound as vq_gemv's low-rank term.
 */
int vq_gemm(const vq_weight *w, const uint16_t *x_bf16, int32_t m, float *y, void *workspace, size_t ws_bytes,
            void *stream);

/* Bytes of workspace vq_gemm needs for this weight and m tokens (0: none).
 * Returns 0 for an invalid descriptor or m < 1 (vq_gemm then reports the
 * error itself).  Host only; touches no device. */
size_t vq_gemm_workspace_size(const vq_weight *w, int32_t m);

/*
 * vq_gemm for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same product and results, with the scratch taken from
 * the library's own static device buffer of VQ_GEMM_NOALLOC_SCRATCH bytes
 * per GPU (held until the process ends; its device address is looked up on
 * the first call on each device).  The caller still passes x and y.
 * Returns VQ_ERR_WORKSPACE, before any HIP call, when the call would need
 * more scratch than that (vq_gemm_workspace_size(w, m) >
 * VQ_GEMM_NOALLOC_SCRATCH: 33 MiB holds fp16 x for 4096 tokens of k_in =
 * 4096 or 2048 tokens of k_in = 8192).
 * Allocates nothing (no hipMalloc or hipFree).  Every call on one GPU shares
 * that GPU's buffer and leaves its contents behind; each call overwrites
 * all of the scratch it reads, so nothing has to be cleared, but calls that
 * overlap in time on one GPU (different streams, different threads) race on
 * it: serialize them.
 */
#define VQ_GEMM_NOALLOC_SCRATCH ((size_t)33 << 20)
int vq_gemm_noalloc(const vq_weight *w, const uint16_t *x_bf16, int32_t m, float *y, void *stream);

/*
 * Randomized Hadamard transform of each row of x (GLQ page, "How it works":
 * random sign flips followed by a fast Walsh-Hadamard transform; "Bit
 * widths": block-diagonal over power-of-two blocks for other sizes):
 *   out[b] = blockdiag(H_n1, H_n2, ...) (signs * x[b]),
 * H_n the orthonormal (1/sqrt(n)) Sylvester-order Hadamard matrix, blocks
 * taken greedily largest first, each at most max_block (28672 with 8192 ->
 * 8192, 8192, 8192, 4096).
 *   x         : [batch][n], VQ_F32 or VQ_BF16
 *   signs     : int8 [n], each +1 or -1
 *   max_block : power of two, 1..16384
 *   out       : float [batch][n]
 * fp32 butterflies; |out - exact| <= (log2(nb) + 2) 2^-24 ||x_block||_2 * 1.01
 * elementwise within each block of size nb.
 */
int rht_apply(const void *x, int32_t x_dtype, int32_t batch, int32_t n, const int8_t *signs,
              int32_t max_block, float *out, void *stream);

/*
 * The transform of rows cut into shards, in one launch (GLQ page,
 * "Inference kernels": the per-shard output transforms of a fused QKV or
 * gate-up layer batched into a single launch; "How it works": the weights
 * are rotated and the inverse transform runs in the inference kernels).
 * Row b of x is n = shard_len[0] + ... + shard_len[n_shards - 1] columns;
 * each shard is transformed on its own, exactly as rht_apply transforms a
 * row of that length (its own greedy block decomposition, the signs of its
 * own columns):
 *   direction VQ_RHT_FORWARD: signs, then the blocks' Hadamard (the input
 *     transform; one shard gives rht_apply);
 *   direction VQ_RHT_INVERSE: the blocks' Hadamard, then signs -- the
 *     inverse (transpose) of the forward transform, the output-side step
 *     y = D H y' for a weight stored rotated on its output side.
 *   x          : [batch][n], VQ_F32 or VQ_BF16, 16-byte aligned
 *   n_shards   : 1..VQ_RHT_MAX_SHARDS
 *   shard_len  : HOST array [n_shards], each >= 1, summing to n; read during
 *                the call only
 *   signs      : int8 [n], each +1 or -1 (device)
 *   max_block  : power of two, 1..16384
 *   out        : float [batch][n], 16-byte aligned; must not alias x
 * Errors (before any HIP call): VQ_ERR_NULL, VQ_ERR_DTYPE, VQ_ERR_VALUE for
 * an unknown direction, VQ_ERR_SHAPE for shard lengths that are not
 * positive or do not sum to n.  Same error bound as rht_apply, per block.
 */
#define VQ_RHT_FORWARD 0
#define VQ_RHT_INVERSE 1
#define VQ_RHT_MAX_SHARDS 16
int rht_apply_shards(const void *x, int32_t x_dtype, int32_t batch, int32_t n, int32_t n_shards,
                     const int32_t *shard_len, const int8_t *signs, int32_t max_block, int32_t direction,
                     float *out, void *stream);

/*
 * The decode-style product with the input transform applied inside the
 * decode kernel (GLQ page, "Advanced", "Trellis codebook": its decode
 * kernels run the input Hadamard transform in every decode block instead of
 * as a separate launch):
 *   y[b] = dequant(W) . RHT(x[b]),  RHT as rht_apply with signs, max_block,
 * for 1..16 tokens, with no buffer for the transformed x: every workgroup
 * transforms its own copy in LDS.  Taken for the weights the 16-bit decode
 * kernels serve, without a sparse or low-rank correction:
 *  - one 16-bit stage, or a 16-bit stage plus one 8- or 16-bit residual
 *    stage, stage scales allowed, with one scale per row, n_out * k_in >= 2^25,
 *    k_in a multiple of 1024 up to 37632 whose 1024-column count is 1, 2, 4
 *    or 8 times one of 1, 2, 4, 7, 8 (the codebook-sliced kernel), or
 *  - a 16-bit first stage, at most one 8- or 16-bit residual stage, stage
 *    scales allowed, K % 2048 == 0 with K <= 32768 (26624 with a 16-bit and
 *    28672 with an 8-bit residual), scale blocks of 32-column units that
 *    divide 2048 or cover the row (the codebook-gather kernel).
 * Any other weight returns VQ_ERR_UNSUPPORTED with nothing launched (use
 * rht_apply, then vq_gemv).  The 8- and 12-bit decode kernel keeps up to
 * 128 KiB of codebooks in LDS; a transform inside it would also need the
 * row of fp32 x there (4 bytes a column), which fits beside two 12-bit
 * codebooks only for rows of up to about 6000 columns.  It is not built:
 * those weights take the separate launch.
 *   x         : [batch][k_in], VQ_F32 or VQ_BF16, 16-byte aligned
 *   signs     : int8 [k_in], each +1 or -1, 16-byte aligned
 *   max_block : power of two, 1..16384 (VQ_ERR_SHAPE otherwise)
 *   y         : float [batch][n_out], 16-byte aligned
 * Same bound as vq_gemv on the transformed x; the transform itself is the
 * fp32 butterfly sequence of rht_apply up to the order of its stages.
 */
int vq_gemv_rht(const vq_weight *w, const void *x, int32_t x_dtype, int32_t batch, const int8_t *signs,
                int32_t max_block, float *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VQMM_H */
