/*
 * nvfp4.h -- C ABI of libnvfp4.so, the NVFP4 4-bit training hot path on AMD MI355X (gfx950).
 *
 * The library quantizes bf16/fp32 tensors to NVFP4, applies the random Hadamard transform to the
 * weight-gradient operands, dequantizes, and multiplies two NVFP4 tensors with fp32
 * accumulation.  An MXFP4 quantizer/GEMM is included as the comparison format.
 *
 * Citation keys for the web pages the operations follow:
 *   [P1] "Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision" (focoia.com.mx)
 *   [P2] "FP4 All the Way: Formacion totalmente cuantificada de LLM" (slashpage.com summary)
 *   [P3] "I ricercatori di Nvidia sbloccano il tutorial LLM a 8 bit che corrisponde alle
 *        prestazioni a 4 bit" (massacarraranews.com)
 *
 * NVFP4 tensor format [P1 Caracteristicas del Formato NVFP4]:
 *   - elements are E2M1 (1 sign, 2 exponent, 1 mantissa bit; values 0, .5, 1, 1.5, 2, 3, 4, 6
 *     with either sign), packed two per byte: element 2j in the low nibble, 2j+1 in the high;
 *   - every block of 16 contiguous elements along the reduction dimension K shares one E4M3
 *     scale byte (OCP E4M3FN, non-negative, at most 448 = 0x7E); 16x16 tiles for weights
 *     [P1 Metodologia: two-dimensional block scaling for weights];
 *   - one fp32 per-tensor decode scale s_dec [P3 Come funziona NVFP4?: multi-level scaling]:
 *     with A the tensor amax, s_dec = A / 2688; the block scale is E4M3(amax_b * 448 / A) and an
 *     element code is E2M1(x * (2688 / A) / scale_b).  The value of a code is v * scale_b * s_dec.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller, 16-byte aligned (GEMM outputs need
 *     only element alignment, and amax / s_dec 4-byte alignment); the library never
 *     allocates or frees memory and keeps no state between calls, so calls on different streams
 *     are independent.  `stream` is a hipStream_t (NULL = the default stream).
 *   - Work is enqueued on `stream` and the call returns without synchronising the host.
 *   - Argument and shape errors return a non-zero status before anything is enqueued.  A kernel
 *     launch failure returns NVFP4_ERR_LAUNCH.  Kernels never trap.
 *   - Inputs must be finite; for NaN/Inf inputs the outputs are unspecified.
 *   - Row strides `ld` are in elements, ld >= cols, and ld * element size must be a multiple of
 *     16 bytes.  Quantized buffers are dense (no stride).
 *   - Size limit of every row-wise call (amax, quantizers, dequantize, sweep): rows * cols / 8
 *     < 2^31, i.e. fewer than 2^34 elements (NVFP4_ERR_SHAPE beyond).  The token-major calls
 *     (Hadamard, dual, transposing MXFP4) take T <= 33553920 tokens (ceil(T / 512) <= 65535
 *     workgroup rows) and F < 2^31 features; nvfp4_quantize_dual also needs its workgroup count
 *     ceil(F / 256) * ceil(T / 256) below 2^31.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

/* Only the functions declared here are exported from the library; everything else it
 * contains (kernels, helpers) is built with hidden visibility. */
#if defined(__GNUC__) || defined(__clang__)
#define NVFP4_API __attribute__((visibility("default")))
#else
#define NVFP4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,     /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = 2,    /* a dimension is negative, not a multiple of the block, or mismatched */
    NVFP4_ERR_DTYPE = 3,    /* unknown dtype or rounding mode */
    NVFP4_ERR_ALIGN = 4,    /* a pointer or row stride is not 16-byte aligned */
    NVFP4_ERR_LAYOUT = 5,   /* a tensor's block layout is not allowed for this call */
    NVFP4_ERR_LAUNCH = 6,   /* the HIP runtime rejected a kernel launch */
    NVFP4_ERR_SCRATCH = 7   /* the call needs more than the library's fixed scratch buffer */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;

/* Forward-pass operands round to nearest (ties to the even code); gradients round
 * stochastically [P2 Describir].  SR rounds |z| up to the next grid value with probability
 * (|z| - lo) / (hi - lo), using a 16-bit uniform from Philox4x32-10 with key = seed and counter
 * = (element index / 8) where the element index is row * cols + col of the OUTPUT tensor; the
 * eight elements of one counter take the 16-bit halves of its four output words in order. */
typedef enum { NVFP4_RNE = 0, NVFP4_SR = 1 } nvfp4_round;

typedef enum {
    NVFP4_BLK_1x16 = 0,     /* scales [rows x cols/16] */
    NVFP4_BLK_16x16 = 1,    /* scales [rows/16 x cols/16] (weights) */
    MXFP4_BLK_1x32 = 2      /* E8M0 scales [rows x cols/32], no per-tensor scale */
} nvfp4_layout;

/* One quantized matrix of logical shape [rows x cols]; cols is the contiguous reduction
 * dimension K.  codes: rows * cols / 2 bytes.  amax / s_dec: one device fp32 each (NVFP4
 * only; the quantizers write both). */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    float *amax;
    float *s_dec;
    int64_t rows;
    int64_t cols;
    int32_t layout;         /* nvfp4_layout */
    int32_t reserved;       /* must be 0 */
} nvfp4_tensor;

/* Human-readable text for a status code (static storage). */
NVFP4_API const char *nvfp4_status_string(nvfp4_status s);

/* Per-tensor amax: *amax_out = max |x| over x [rows x cols] (row stride ld).  This is the first
 * level of the two-level scaling [P3 Come funziona NVFP4?].  amax_out is overwritten.
 * cols % 8 == 0 (the pass reads 8 elements at a time), else NVFP4_ERR_SHAPE; every NVFP4
 * tensor satisfies it (cols % 16 == 0). */
NVFP4_API nvfp4_status nvfp4_amax(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                                  float *amax_out, void *stream);

/* amax of the random-Hadamard-transformed tensor (see nvfp4_hadamard_quantize), without
 * writing the transform: x is [T tokens x F features], T % 16 == 0 and F % 8 == 0 (else
 * NVFP4_ERR_SHAPE). */
NVFP4_API nvfp4_status nvfp4_hadamard_amax(const void *x, nvfp4_dtype dt, int64_t T, int64_t F, int64_t ld,
                                           uint64_t sign_seed, float *amax_out, void *stream);

/* Accumulating forms of nvfp4_amax and nvfp4_hadamard_amax [P3 Come funziona NVFP4?: the
 * per-tensor level of the scaling]: *amax_inout = max(*amax_inout, amax) with the same amax as
 * above, and no zero-fill of *amax_inout first.  The caller initialises *amax_inout (0 gives the
 * amax of x alone), which lets one amax cover several tensors or micro-batches and lets a caller
 * clear many amax slots in one operation instead of one launch per slot.  *amax_inout must hold
 * a non-negative, non-NaN float (it is raised by an unsigned atomic max on its bit pattern).  An
 * empty x leaves it unchanged.  Same shape rules and errors as the non-accumulating calls:
 * cols % 8 == 0 for nvfp4_amax_accumulate, T % 16 == 0 and F % 8 == 0 for the Hadamard form. */
NVFP4_API nvfp4_status nvfp4_amax_accumulate(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                             int64_t ld, float *amax_inout, void *stream);
NVFP4_API nvfp4_status nvfp4_hadamard_amax_accumulate(const void *x, nvfp4_dtype dt, int64_t T, int64_t F,
                                                      int64_t ld, uint64_t sign_seed, float *amax_inout,
                                                      void *stream);

/* 1D NVFP4 quantization of x [out->rows x out->cols] (row stride ld) into `out`
 * (layout NVFP4_BLK_1x16, cols % 16 == 0) [P1 Caracteristicas; P2 Describir].
 * amax_in: device pointer to the tensor amax to use, or NULL to compute it first (two passes).
 * Writes out->codes, out->scales, *out->amax (= the amax used) and *out->s_dec. */
NVFP4_API nvfp4_status nvfp4_quantize_1d(const void *x, nvfp4_dtype dt, int64_t ld, const float *amax_in,
                                         nvfp4_round rnd, uint64_t seed, const nvfp4_tensor *out,
                                         void *stream);

/* nvfp4_quantize_1d plus, in the same pass, the quantization-noise diagnostic of
 * [P2 Describir: quantized training loses efficiency once the gradient norm falls below about
 * sqrt(3) times the quantization noise]: sums[0] = sum of x^2 and sums[1] = sum of (Q(x) - x)^2
 * over the tensor, Q(x) the dequantized value (as nvfp4_dequantize computes it in fp32).  The
 * gradient norm is sqrt(sums[0]), the noise sqrt(sums[1]); the caller compares their ratio with
 * sqrt(3).  sums: device, two doubles, 8-byte aligned, overwritten.  Accumulated in fp32 per
 * 16-element block (on values times s_enc = 2688 / amax) and in fp64 across blocks, with device
 * atomics: the order of the additions, and so the last bits of the sums, vary from run to run;
 * codes and scales are exactly those of nvfp4_quantize_1d.  A tensor treated as zero (amax below
 * 2^-100) reports sums of its fp32 squares, which may underflow to 0. */
NVFP4_API nvfp4_status nvfp4_quantize_1d_noise(const void *x, nvfp4_dtype dt, int64_t ld, const float *amax_in,
                                               nvfp4_round rnd, uint64_t seed, const nvfp4_tensor *out,
                                               double *sums, void *stream);

/* 2D NVFP4 quantization of a weight w [out->rows x out->cols] with one E4M3 scale per 16x16
 * tile, round to nearest [P1 Metodologia: two-dimensional block scaling for weights].
 * out: layout NVFP4_BLK_16x16, rows % 16 == cols % 16 == 0.  out_t (optional, may be NULL):
 * the same quantized values transposed, [cols x rows], layout NVFP4_BLK_16x16 -- the dgrad
 * operand.  Both share amax and s_dec values (out_t's amax/s_dec pointers are written too if
 * they are non-NULL). */
NVFP4_API nvfp4_status nvfp4_quantize_2d(const void *w, nvfp4_dtype dt, int64_t ld, const float *amax_in,
                                         const nvfp4_tensor *out, const nvfp4_tensor *out_t, void *stream);

/* Random Hadamard transform + transpose + 1D quantization of a wgrad operand
 * [P1 Metodologia: random Hadamard transforms].  x is [T tokens x F features] (row stride ld);
 * each 16-token chunk of each feature column is replaced by (1/4) H16 D x, with H16 the
 * Sylvester Hadamard matrix and D = diag(d), d_j = -1 iff bit j of word 0 of
 * Philox4x32-10(key = sign_seed, counter = 0) is set.  The result is written feature-major:
 * out is [F x T] (out->rows = F, out->cols = T, layout NVFP4_BLK_1x16), so the token dimension
 * is the contiguous K of the wgrad GEMM and each 16-token chunk is one NVFP4 block.
 * T % 16 == 0 and F % 8 == 0 (a thread transforms 8 adjacent features), else NVFP4_ERR_SHAPE.
 * amax_in: the amax of the TRANSFORMED tensor, or NULL to compute it. */
NVFP4_API nvfp4_status nvfp4_hadamard_quantize(const void *x, nvfp4_dtype dt, int64_t ld, uint64_t sign_seed,
                                               const float *amax_in, nvfp4_round rnd, uint64_t seed,
                                               const nvfp4_tensor *out, void *stream);

/* nvfp4_hadamard_quantize plus, in the same pass, the quantization-noise diagnostic of
 * [P2 Describir: quantized training loses efficiency once the gradient norm falls below about
 * sqrt(3) times the quantization noise] for the tensor this call encodes, the transformed
 * y = (1/4) H16 D x: sums[0] = sum of y^2 and sums[1] = sum of (Q(y) - y)^2, Q(y) the dequantized
 * value (as nvfp4_dequantize computes it in fp32).  Since (1/4) H16 D is orthogonal, sum y^2
 * equals sum x^2 up to rounding.  sums: device, two doubles, 8-byte aligned, overwritten.
 * Accumulated as in nvfp4_quantize_1d_noise (fp32 per 16-element block on values times s_enc,
 * fp64 across blocks, device atomics: the last bits vary from run to run); codes and scales are
 * exactly those of nvfp4_hadamard_quantize.  Shape rules as nvfp4_hadamard_quantize. */
NVFP4_API nvfp4_status nvfp4_hadamard_quantize_noise(const void *x, nvfp4_dtype dt, int64_t ld,
                                                     uint64_t sign_seed, const float *amax_in,
                                                     nvfp4_round rnd, uint64_t seed,
                                                     const nvfp4_tensor *out, double *sums, void *stream);

/* amax of x [T x F] and of its random Hadamard transform (as in nvfp4_hadamard_quantize) in one
 * read of x: *amax_out = max |x|, *amax_t_out = max |(1/4) H16 D x|.  T % 16 == 0, F % 8 == 0;
 * the two outputs must be distinct (else NVFP4_ERR_SHAPE). */
NVFP4_API nvfp4_status nvfp4_dual_amax(const void *x, nvfp4_dtype dt, int64_t T, int64_t F, int64_t ld,
                                       uint64_t sign_seed, float *amax_out, float *amax_t_out, void *stream);

/* Accumulating form of nvfp4_dual_amax [P3 Come funziona NVFP4?: the per-tensor level of the
 * scaling]: *amax_inout = max(*amax_inout, max |x|) and *amax_t_inout = max(*amax_t_inout,
 * max |(1/4) H16 D x|), with no zero-fill first, as nvfp4_amax_accumulate: the caller initialises
 * both (0 gives the amaxes of x alone), so that one operation can clear every amax slot of a
 * training step.  Both must hold non-negative, non-NaN floats and be distinct; an empty x leaves
 * them unchanged.  Shape rules and errors as nvfp4_dual_amax. */
NVFP4_API nvfp4_status nvfp4_dual_amax_accumulate(const void *x, nvfp4_dtype dt, int64_t T, int64_t F,
                                                  int64_t ld, uint64_t sign_seed, float *amax_inout,
                                                  float *amax_t_inout, void *stream);

/* Fused dual-orientation quantization: one read of an activation or gradient x [T tokens x
 * F features] (row stride ld) writes both NVFP4 copies a training step takes from it
 * [P2 Describir: all three GEMMs on FP4 operands; P1 Metodologia: random Hadamard transforms on
 * the weight-gradient operands]:
 *   out   [T x F], layout 1x16: the row-wise copy (fprop / dgrad operand), bit-identical to
 *         nvfp4_quantize_1d(x, dt, ld, amax_in, rnd, seed, out);
 *   out_t [F x T], layout 1x16: the Hadamard-transformed transposed copy (wgrad operand),
 *         bit-identical to nvfp4_hadamard_quantize(x, dt, ld, sign_seed, amax_t_in, rnd, seed_t,
 *         out_t).
 * amax_in / amax_t_in: the amax of x and of its transform, or NULL to compute that one first
 * (both NULL: one fused pass as nvfp4_dual_amax into out->amax and out_t->amax; only amax_t_in
 * NULL: the transform's amax into out_t->amax; only amax_in NULL: nvfp4_amax into out->amax).
 * A supplied amax is never overwritten before it is used, even when it is out's own slot.
 * Requirements:
 * T % 16 == 0, F % 16 == 0; out and out_t have distinct amax and s_dec pointers. */
NVFP4_API nvfp4_status nvfp4_quantize_dual(const void *x, nvfp4_dtype dt, int64_t ld, uint64_t sign_seed,
                                           const float *amax_in, const float *amax_t_in, nvfp4_round rnd,
                                           uint64_t seed, uint64_t seed_t, const nvfp4_tensor *out,
                                           const nvfp4_tensor *out_t, void *stream);

/* Dequantize an NVFP4 tensor (1x16 or 16x16): y = fl(fl(v * scale_b) * s_dec) in fp32, stored
 * as fp32 or rounded to nearest-even bf16.  y is [q->rows x q->cols], row stride ld. */
NVFP4_API nvfp4_status nvfp4_dequantize(const nvfp4_tensor *q, void *y, nvfp4_dtype dt, int64_t ld,
                                        void *stream);

/* NVFP4 x NVFP4 GEMM with fp32 accumulation [P2 Describir: weights, activations and gradients
 * all in FP4]: C = A * B^T, A [M x K] (layout 1x16), B [N x K] (layout 1x16 or 16x16),
 *   C[m,n] = s_dA * s_dB * sum_k (vA * sA) * (vB * sB),
 * stored fp32 or bf16 (round to nearest even) into c [M x N] with row stride ldc.
 * Requirements: a->cols == b->cols == K, K % 16 == 0; c need only be element-aligned.
 * K == 0 writes zeros (the empty sum) and reads neither operand's codes nor scales. */
NVFP4_API nvfp4_status nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, nvfp4_dtype c_dt,
                                  int64_t ldc, void *stream);

/* Bytes of workspace with which nvfp4_gemm_ws splits an M x N x K GEMM on the current device
 * (see there); 0 when it would not split (the last round of 256 x 256 output tiles over the
 * device's compute units is empty or more than half full, K % 64 != 0, or K too short for
 * splits of at least 16 steps of 64).  At most 64 MiB (256 partial tiles of 256 KiB).  Negative
 * or >= 2^31 dimensions: NVFP4_ERR_SHAPE; bytes NULL: NVFP4_ERR_NULL. */
NVFP4_API nvfp4_status nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, size_t *bytes);

/* nvfp4_gemm with a caller-owned device workspace [P2 Describir: all three GEMMs on FP4
 * operands].  The output is cut into 256 x 256 tiles, one per workgroup, which the device runs
 * in rounds of one tile per compute unit.  When the last round is at most half full, each of its
 * tiles is split along K into 2..8 parts: the parts run as separate workgroups that write their
 * unscaled fp32 sums to the workspace, and a second kernel adds a tile's parts in part order,
 * applies s_dA * s_dB and stores C.  The result is deterministic, within the same bound of the
 * exact sum as nvfp4_gemm's, but its last bits can differ from nvfp4_gemm's for the split tiles
 * (another fp32 addition order).  workspace: device, 16-byte aligned, ws_bytes of it usable;
 * with NULL or fewer bytes than nvfp4_gemm_workspace_size this call is exactly nvfp4_gemm.  Its
 * contents on return are unspecified; calls that may overlap in time need distinct workspaces.
 * Shapes, layouts and errors as nvfp4_gemm; a misaligned workspace: NVFP4_ERR_ALIGN. */
NVFP4_API nvfp4_status nvfp4_gemm_ws(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, nvfp4_dtype c_dt,
                                     int64_t ldc, void *workspace, size_t ws_bytes, void *stream);

/* nvfp4_gemm_ws for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid allocation): the split partial tiles go to a scratch
 * array that the library holds in device memory, 64 MiB per device (256 partial tiles of 256 x
 * 256 fp32), from the first call on a device until the process ends.  Same result as nvfp4_gemm_ws
 * with a large enough workspace, bit for bit.  A shape whose split needs more than 64 MiB (only
 * possible on a device with more than 256 compute units) returns NVFP4_ERR_SCRATCH and enqueues
 * nothing; a failed lookup of the array's device address returns NVFP4_ERR_LAUNCH.  Every call
 * on one device shares that device's array: calls that overlap in time on one device (other
 * streams, other host threads) race and must be ordered by the caller.  Allocates nothing. */
NVFP4_API nvfp4_status nvfp4_gemm_ws_noalloc(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c,
                                             nvfp4_dtype c_dt, int64_t ldc, void *stream);

/* Format sweep [P2 Describir: block size, scale format and rounding method are the FP4 design
 * choices explored, and 16-element blocks with E4M3 scales (NVFP4) come out best]: quantize
 * x [rows x cols] (row stride ld) with `block` (8, 16 or 32) elements per scale along the row and
 * the scale format `scale_fmt`
 *   0: E4M3 block scale under the fp32 per-tensor scale (the NVFP4 steps),
 *   1: E8M0 power-of-two scale 2^(floor(log2 amax_b) - 2), no tensor scale (the MXFP4 steps),
 * round RNE or SR (element index row * cols + col), and write the dequantized fp32 values to y
 * (row stride ldy, 16-byte aligned rows).  No codes are kept: this measures formats.  Block 16 /
 * format 0 reproduces nvfp4_dequantize of nvfp4_quantize_1d; block 32 / format 1 that of
 * mxfp4_quantize_1d.  amax_in (format 0 only): the tensor amax, or NULL to compute it into
 * *amax_out, which is then required.  amax_out (optional): the amax used (0 for format 1).
 * sums (optional, two doubles, overwritten): sum x^2 and sum (y - x)^2, accumulated in fp64 with
 * device atomics (run-dependent order in the last bits).  Unknown block or format:
 * NVFP4_ERR_SHAPE / NVFP4_ERR_DTYPE. */
NVFP4_API nvfp4_status nvfp4_qdq(const void *x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                                 int32_t block, int32_t scale_fmt, const float *amax_in, nvfp4_round rnd,
                                 uint64_t seed, float *y, int64_t ldy, float *amax_out, double *sums,
                                 void *stream);

/* MXFP4 quantization (the comparison format of [P3 NVFP4 in pratica]): 32-element blocks along
 * cols with an E8M0 scale 2^(floor(log2 amax_b) - 2) (byte = exponent + 127, clamped to
 * [0, 254]; an all-zero block gets byte 127); codes E2M1 of x * 2^-exponent, RNE or SR as above.
 * out: layout MXFP4_BLK_1x32, cols % 32 == 0; amax/s_dec are not used. */
NVFP4_API nvfp4_status mxfp4_quantize_1d(const void *x, nvfp4_dtype dt, int64_t ld, nvfp4_round rnd,
                                         uint64_t seed, const nvfp4_tensor *out, void *stream);

/* MXFP4 quantization of x^T, for the wgrad operands of the MXFP4 comparison [P3 NVFP4 in
 * pratica]: x [T tokens x F features] (row stride ld) is read once and out [F x T] (layout
 * MXFP4_BLK_1x32, out->rows = F, out->cols = T) receives, for every feature, its T values in
 * 32-token blocks -- the same bytes as mxfp4_quantize_1d of the transposed matrix, SR element
 * index feature * T + token included.  No Hadamard transform (that is part of the NVFP4 recipe).
 * T % 32 == 0, F % 8 == 0 (else NVFP4_ERR_SHAPE); the grid limits of nvfp4_hadamard_quantize
 * apply. */
NVFP4_API nvfp4_status mxfp4_quantize_1d_t(const void *x, nvfp4_dtype dt, int64_t ld, nvfp4_round rnd,
                                           uint64_t seed, const nvfp4_tensor *out, void *stream);

/* Both MXFP4 copies of x from one read, for the MXFP4 comparison [P3 NVFP4 in pratica]: x [T x F]
 * (row stride ld) gives out [T x F] (out->rows = T, out->cols = F), the same bytes as
 * mxfp4_quantize_1d(x, rnd, seed), and out_t [F x T], the same bytes as
 * mxfp4_quantize_1d_t(x, rnd, seed_t).  Both tensors caller-owned, layout MXFP4_BLK_1x32.
 * T % 32 == 0 and F % 32 == 0 (else NVFP4_ERR_SHAPE); the workgroup count
 * ceil(F / 256) * ceil(T / 256) (RNE) or ceil(F / 256) * ceil(T / 128) (SR) must stay below
 * 2^31, and the token-major limits above apply. */
NVFP4_API nvfp4_status mxfp4_quantize_dual(const void *x, nvfp4_dtype dt, int64_t ld, nvfp4_round rnd,
                                           uint64_t seed, uint64_t seed_t, const nvfp4_tensor *out,
                                           const nvfp4_tensor *out_t, void *stream);

/* MXFP4 x MXFP4 GEMM, C = A * B^T with fp32 accumulation, both operands MXFP4_BLK_1x32, stored
 * fp32 or bf16 (round to nearest even) into c [M x N] with row stride ldc.  Requirements as for
 * nvfp4_gemm with K % 32 == 0 (s_dec and amax are not used); K == 0 writes zeros. */
NVFP4_API nvfp4_status mxfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, nvfp4_dtype c_dt,
                                  int64_t ldc, void *stream);

/* Bytes of workspace with which mxfp4_gemm_ws splits an M x N x K GEMM on the current device (0:
 * no split; only K % 256 == 0 GEMMs split, in parts of at least 4 steps of 256).  At most
 * 64 MiB.  Errors as nvfp4_gemm_workspace_size. */
NVFP4_API nvfp4_status mxfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, size_t *bytes);

/* mxfp4_gemm with a caller-owned device workspace, splitting a partly empty last round of output
 * tiles along K exactly as nvfp4_gemm_ws does [P3 NVFP4 in pratica: the comparison format gets
 * the same GEMM schedule]: deterministic, bit-for-bit different from mxfp4_gemm only in the fp32
 * addition order of the split tiles; with NULL or too small a workspace exactly mxfp4_gemm.
 * Workspace rules as nvfp4_gemm_ws. */
NVFP4_API nvfp4_status mxfp4_gemm_ws(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, nvfp4_dtype c_dt,
                                     int64_t ldc, void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
