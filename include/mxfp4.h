/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) W4A4 MXFP4 linear-layer library.
 *
 * A W4A4 MXFP4 linear layer Y = X * W^T has two device steps:
 *   1. mxfp4_quantize_rotate: online activation quantization.  Each row of X
 *      is cut into 32-element blocks along K; each block is optionally
 *      rotated (a normalized Hadamard-32 or a Kronecker-factored 32x32
 *      transform), then shares one power-of-two E8M0 scale and is encoded as
 *      4-bit E2M1 codes, two per byte.
 *   2. mxfp4_gemm: a GEMM that reads the packed MXFP4 operands directly (no
 *      dequantize pass), accumulates in fp32 and writes fp32 or bf16.
 * Weights are quantized once, offline, with the same quantizer (the weight
 * side of a rotation: the same Hadamard-32, or the inverse-transpose
 * Kronecker factors from mxfp4_inverse_transpose).
 *
 * Sources (page titles and sections as the pages give them):
 *  - "AMD Quark delivers MXFP4 quantization for FLUX.1-dev on Instinct MI350
 *    with 1.92x speedup": "What is MXFP4 and why does it eliminate
 *    dequantization overhead?" (32-element blocks sharing one scale, 4-bit
 *    elements, the MX specification) and "MXFP4 quantization for diffusion
 *    models" (the GEMM consumes MXFP4 directly, no dequantization phase).
 *  - "Bridging the Gap Between Promise and Performance for Microscaling FP4
 *    Quantization": "Probleemstelling" (group size 32, power-of-two E8M0
 *    scales), "Methodologie: MR-GPTQ" item 1 (block-wise Hadamard on weights
 *    and activations), "GPU Kernel Ondersteuning (QuTLASS)" (the rotation runs
 *    online inside the quantization kernel).
 *  - "KroQuant: Effiziente Post-Training-Quantisierung fuer Diffusion
 *    Transformers mittels Kronecker-Produkt-Struktur": abstract and
 *    "Tiefenanalyse" (learned Kronecker-structured transform on each
 *    32-element activation block), "Hintergrund" (the inverse transform goes
 *    on the weights, offline).
 *
 * Conventions shared by every entry point:
 *  - Device pointers are HIP device memory owned by the caller; the library
 *    allocates nothing and keeps no mutable global state (calls are
 *    re-entrant).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *    enqueued on it and the call returns without synchronizing; device faults
 *    surface at the caller's next synchronization, as usual in HIP.
 *  - Argument checks are synchronous and nothing is launched when they fail.
 *    No exception crosses the ABI and the library never aborts.
 *
 * Packed layouts.  Both operands of a GEMM use the same layout.
 *  MXFP4_LAYOUT_ROWMAJOR (the interchange format; K contiguous, "K-major"):
 *  - codes [rows][K/2] uint8: element 2j of a row in the low nibble of byte j,
 *    element 2j+1 in the high nibble.  E2M1 code = sign<<3 | magnitude index
 *    into {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *  - scales [rows][K/32] uint8: E8M0 byte s of block b means 2^(s-127).
 *  Both are dense (row strides K/2 and K/32 bytes).
 *  MXFP4_LAYOUT_TILED (the GEMM-native format; K a multiple of 128): rows are
 *  grouped in tiles of 256 and K in stages of 128 elements (4 blocks).
 *  With T = ceil(rows / 256) and S = K / 128:
 *  - codes [T][S][256][64] bytes: in tile t, stage s, row r (global row
 *    256 t + r), block 4 s + c (c = 0..3) occupies the 16 bytes at
 *    r * 64 + 16 * (c ^ ((r >> 1 ^ r >> 2) & 3)), with the row-major nibble
 *    order inside the block;
 *  - scales [T][S][256][4] bytes: the scale of block 4 s + c of row r at r * 4 + c.
 *  Rows rows .. 256 T - 1 are padding.  Their content is unspecified: each
 *  output element of the GEMM depends on one real row of each operand only,
 *  so padding never reaches a stored result, whatever it holds (NaN scale
 *  bytes included).  The quantizer writes zero codes and scales into the
 *  padding rows of the last 16-row group that holds real rows and leaves the
 *  rest of the buffer untouched.  Every load
 *  the GEMM makes of a tiled operand is then a contiguous 1 KiB (codes) or
 *  256-byte (scales) run.  mxfp4_tiled_bytes gives the buffer sizes.
 *
 * Quantizer rule (per 32-block, after the optional rotation, all in fp32):
 *  amax = max |y_i|;  e = max(floor(log2 amax) - 2, -127), e = -127 for
 *  amax = 0;  scale byte = e + 127;  code_i = sign(y_i) | RNE-saturating
 *  E2M1 index of |y_i| * 2^-e (ties to the even mantissa, > 6 saturates to 6;
 *  the sign bit is kept for values that round to zero).
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(_WIN32)
#define MXFP4_API
#else
#define MXFP4_API __attribute__((visibility("default")))
#endif

/* Status codes returned by every entry point. */
typedef enum {
    MXFP4_OK = 0,
    MXFP4_ERR_INVALID_ARG = 1,  /* null pointer, bad size/stride, bad enum */
    MXFP4_ERR_UNSUPPORTED = 2,  /* valid request the library does not run
                                   (misaligned pointer, size beyond limits) */
    MXFP4_ERR_HIP = 3           /* a HIP runtime call or launch failed */
} mxfp4_status;

/* Element types of dense inputs and outputs. */
typedef enum {
    MXFP4_F32 = 0,
    MXFP4_BF16 = 1
} mxfp4_dtype;

/* Block transform applied before quantization. */
typedef enum {
    MXFP4_ROT_NONE = 0,        /* plain MXFP4 round-to-nearest */
    MXFP4_ROT_HADAMARD32 = 1,  /* y = H32 x / sqrt(32), Sylvester order */
    MXFP4_ROT_KRON = 2,        /* y = (A (x) B) x, A p x p, B q x q, p*q=32 */
    MXFP4_ROT_SMOOTH = 3       /* y[c] = x[c] * a[c], per-channel factors */
} mxfp4_rot_kind;

/* Memory layout of packed codes and scales (see "Packed layouts" above). */
typedef enum {
    MXFP4_LAYOUT_ROWMAJOR = 0,
    MXFP4_LAYOUT_TILED = 1
} mxfp4_layout;

/* Rotation descriptor (host struct; read during the call).
 * HADAMARD32 evaluation order (fp32, no fused ops): butterflies
 *   (u, v) -> (u + v, u - v) with strides 1, 2, 4, 8, 16, then a multiply by
 *   fp32(1/sqrt(32)) = 0x3E3504F3.
 * KRON evaluation order: with Xm[j][l] = x[q*j + l],
 *   U[j][k] = chain_l B[k][l] * Xm[j][l],  y[q*i + k] = chain_j A[i][j] * U[j][k],
 *   where a chain is the rounded first product followed by fused
 *   multiply-adds in ascending index order.
 * SMOOTH: per-channel smoothing, the SmoothQuant-style baseline that
 *   "KroQuant: ..." compares its transform with: column c of the input is
 *   multiplied by a[c] (one fp32 multiply; a[c] = 1/s[c] divides by the
 *   smoothing factor s[c], and the weights take a[c]^-1 = s[c]).  `a` holds
 *   k factors, the k of the call.  Calibrating the factors is the caller's.  */
typedef struct {
    int32_t kind;      /* mxfp4_rot_kind */
    int32_t p;         /* KRON: rows of A (1, 2, 4, 8, 16 or 32) */
    int32_t q;         /* KRON: rows of B, p * q == 32 */
    int32_t reserved;  /* must be 0 */
    const float* a;    /* KRON: device pointer, p*p fp32 row-major;
                          SMOOTH: device pointer, k fp32 factors, 16-byte aligned */
    const float* b;    /* KRON: device pointer, q*q fp32 row-major */
} mxfp4_rotation;

/* Online quantization of a dense matrix to MXFP4 (with optional rotation).
 *   x       device, [rows][ld_x] elements of x_dtype (F32 or BF16); the first
 *           k columns of each row are quantized.  16-byte aligned, and ld_x a
 *           multiple of 8 (BF16) or 4 (F32), else MXFP4_ERR_UNSUPPORTED.
 *   rows    >= 0 (0 is a no-op);  k > 0, multiple of 32 (of 128 for TILED);
 *           ld_x >= k.
 *   rot     NULL or kind NONE: no rotation.
 *   layout  mxfp4_layout of the outputs.
 *   codes   device, 16-byte aligned (written): [rows][k/2] bytes (ROWMAJOR),
 *           or the tiled codes, sized for the padding rows (TILED; see the
 *           layout above for what is written there).
 *   scales  device (written): [rows][k/32] bytes (ROWMAJOR), or the tiled
 *           scales (TILED, 4-byte aligned).
 * Errors: INVALID_ARG for null pointers (when rows > 0), k % 32 != 0 (k % 128
 *   for TILED), k <= 0, rows < 0, ld_x < k, bad dtype or layout, bad rotation
 *   (unknown kind, p*q != 32, null factor pointers); UNSUPPORTED for
 *   misalignment or rows * k / 32 >= 2^31; HIP if the launch fails. */
MXFP4_API mxfp4_status mxfp4_quantize_rotate(const void* x, int32_t x_dtype,
                                             int64_t rows, int64_t k, int64_t ld_x,
                                             const mxfp4_rotation* rot, int32_t layout,
                                             uint8_t* codes, uint8_t* scales,
                                             void* stream);

/* Scale-fitted quantization, for the offline weight side: as
 * mxfp4_quantize_rotate, but each block's E8M0 exponent is the one of
 * e0 - 1, e0, e0 + 1 (e0 the rule above) whose encoding has the smallest
 * squared error against the transformed block -- each error summed in binary64
 * over the 32 elements in order as s = s + (v - x_hat)^2, ties keeping e0,
 * then e0 + 1 ("Bridging the Gap Between Promise and Performance for
 * Microscaling FP4 Quantization", "Methodologie: MR-GPTQ" item 2 fits the
 * MXFP4 scale exponent to the data; the candidate set and the error are this
 * library's reading).  Same arguments and errors as mxfp4_quantize_rotate. */
MXFP4_API mxfp4_status mxfp4_quantize_fit(const void* x, int32_t x_dtype,
                                          int64_t rows, int64_t k, int64_t ld_x,
                                          const mxfp4_rotation* rot, int32_t layout,
                                          uint8_t* codes, uint8_t* scales,
                                          void* stream);

/* Y = A * B^T on MXFP4 operands, fp32 accumulation.
 *   a_codes/a_scales  device, A (m rows) in `layout`.
 *   b_codes/b_scales  device, B (n rows) in `layout`
 *                     (for a linear layer B = W, [out_features][in_features]).
 *   m, n >= 0 (0 is a no-op), k > 0 multiple of 32 (of 128 for TILED).
 *   y       device, [m][ld_y] elements of y_dtype (F32 or BF16), ld_y >= n;
 *           element (i, j) = sum over blocks of 2^(sa-127) 2^(sb-127) times
 *           the block's E2M1 dot product, accumulated in fp32, rounded to
 *           bf16 (nearest-even) for BF16 output.
 *   Code pointers 16-byte aligned; TILED scale pointers 4-byte aligned.
 * Limits: with TILED operands and m > 64, each operand's tiled code bytes
 *   (256 * ceil(rows / 256) * k / 2) must stay below 2^32.
 * Errors: INVALID_ARG for null pointers (when m, n > 0), k % 32 != 0 (k % 128
 *   for TILED), k <= 0, negative sizes, ld_y < n, bad dtype or layout;
 *   UNSUPPORTED for misaligned pointers, m, n, k >= 2^30, or TILED operands
 *   past the code-byte limit above; HIP if the launch fails. */
MXFP4_API mxfp4_status mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m,
                                  const uint8_t* b_codes, const uint8_t* b_scales, int64_t n,
                                  int64_t k, int32_t layout, void* y, int32_t y_dtype, int64_t ld_y,
                                  void* stream);

/* Y = A * B^T with an MXFP4 output: the GEMM's fp32 result is requantized in
 * the epilogue, per 32-element block along N (the next layer's K), by the
 * quantizer's rule (E8M0 from the block amax, RNE-saturating E2M1 codes; no
 * rotation), so the next layer reads MXFP4 activations without a bf16 round
 * trip.  The epilogue runs in the kernel that mxfp4_gemm takes for the same
 * operands (the decode kernel for m <= 64, the large-tile kernel above), on
 * the same fp32 sums: the codes and scales equal mxfp4_quantize_rotate
 * applied to mxfp4_gemm's fp32 Y, bit for bit.  This is a reading of "AMD
 * Quark delivers MXFP4 quantization for FLUX.1-dev ...", "MXFP4 quantization
 * for diffusion models": the MXFP4 kernel hands on its result with no
 * FP16/BF16 conversion in between.
 *   a_*, b_*, m, n, k, layout  as for mxfp4_gemm; k a multiple of 128.
 *   y_codes/y_scales  device (written): Y in `y_layout` -- ROWMAJOR
 *           [m][n/2] and [m][n/32], or TILED with m rows (padding rows not
 *           written).  16-byte aligned codes, 4-byte aligned scales.
 * Errors: INVALID_ARG for null pointers (when m, n > 0), bad layouts, k <= 0
 *   or k % 32 (k % 128 for TILED operands), negative sizes; UNSUPPORTED for
 *   n % 32 != 0 (n % 128 for a TILED output), k % 128 != 0, misaligned
 *   pointers, sizes >= 2^30, or operands past the code-byte limit of
 *   mxfp4_gemm (m > 64); HIP if the launch fails. */
MXFP4_API mxfp4_status mxfp4_gemm_requant(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m,
                                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t n,
                                          int64_t k, int32_t layout, uint8_t* y_codes, uint8_t* y_scales,
                                          int32_t y_layout, void* stream);

/* Fused small-M linear layer Y = Q(rot(X)) * W^T for decode shapes, in one
 * kernel launch: the activations are rotated and quantized inside the GEMM
 * kernel, and the weights start streaming from HBM while that happens.  The
 * rotation "fused into the quantization and matmul kernels" is the design of
 * "Bridging the Gap Between Promise and Performance for Microscaling FP4
 * Quantization", "GPU Kernel Ondersteuning (QuTLASS)".  A few workgroups
 * quantize X into the workspace (1152 bytes per 16 rows and 128 columns, in
 * the matrix cores' operand order) and the others wait for them on a
 * device-scope counter.  The quantized activations equal
 * mxfp4_quantize_rotate's bit for bit, and Y equals mxfp4_quantize_rotate
 * followed by mxfp4_gemm bit for bit (the same K split and summation order).
 *   x       device, [m][ld_x] BF16 activations, 16-byte aligned, ld_x a
 *           multiple of 8, ld_x >= k.
 *   rot     NULL / NONE, HADAMARD32, SMOOTH, or KRON with 2 <= p <= 16.
 *   w_codes/w_scales  device, W (n rows, pre-quantized) in `layout`.
 *   m       1 <= m <= 64 (0 is a no-op); n >= 0; k > 0 multiple of 32 (of
 *           128 for TILED).
 *   y       device, [m][ld_y] of y_dtype (F32 or BF16), ld_y >= n.
 *   workspace, workspace_bytes  device scratch of at least
 *           mxfp4_linear_small_workspace(m, n, k) bytes, 256-byte aligned.
 *           Its first 4 KiB hold the handoff counters, the same region for
 *           every shape.  They must be zero before the workspace's first use
 *           (e.g. one hipMemset), and every call leaves them zero when its
 *           kernel completes, so one workspace serves calls of any shape in
 *           stream order.  The 32-bit word at byte 2048 of that region is
 *           set to a nonzero value if a workgroup ever stopped waiting for
 *           the quantized activations at its bound (2^20 polls, tens of
 *           milliseconds; then that call's Y is undefined); no call clears
 *           it.  Calls that may run at the same time (other streams, other
 *           host threads) need workspaces of their own.
 * Errors: INVALID_ARG as for mxfp4_quantize_rotate and mxfp4_gemm, and for a
 *   missing or short workspace; UNSUPPORTED for m > 64, F32 activations, a
 *   KRON rotation with p = 1 or p = 32, misaligned pointers (use
 *   mxfp4_quantize_rotate + mxfp4_gemm there), or a workspace image of
 *   2 GiB or more; HIP if the launch fails. */
MXFP4_API mxfp4_status mxfp4_linear_small(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                          int64_t ld_x, const mxfp4_rotation* rot,
                                          const uint8_t* w_codes, const uint8_t* w_scales, int64_t n,
                                          int32_t layout, void* y, int32_t y_dtype, int64_t ld_y,
                                          void* workspace, int64_t workspace_bytes, void* stream);

/* mxfp4_linear_small for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and result as mxfp4_linear_small without the
 * workspace: the workspace is a fixed 4 MiB array of device memory inside
 * the library instead (one per GPU, held until the process ends; its
 * counters are cleared by the first call on each device).  The call
 * allocates nothing.  Every call on a GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (other streams, other host threads) race:
 * serialize them, or give each its own workspace with mxfp4_linear_small.
 * Limit: mxfp4_linear_small_workspace(m, n, k) <= 4 MiB (k <= 465536 for
 * m <= 16, k <= 116352 for m <= 64).
 * Errors: as mxfp4_linear_small, and UNSUPPORTED past that limit (checked
 *   before anything is launched); HIP if the scratch address lookup or a
 *   launch fails. */
MXFP4_API mxfp4_status mxfp4_linear_small_noalloc(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                                  int64_t ld_x, const mxfp4_rotation* rot,
                                                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t n,
                                                  int32_t layout, void* y, int32_t y_dtype, int64_t ld_y,
                                                  void* stream);

/* Workspace size of mxfp4_linear_small for (m, n, k): 0 when m or n is 0,
 * else 4 KiB of counters plus 1152 ceil(m / 16) ceil(k / 128) bytes for the
 * quantized activations (40 960 bytes for 16 x 4096 -> 14336).
 * Errors: INVALID_ARG for a null pointer, negative sizes, k not a positive
 *   multiple of 32; UNSUPPORTED for m > 64, n or k >= 2^30, or an
 *   activation image of 2 GiB or more (mxfp4_linear_small returns
 *   UNSUPPORTED for the same shapes). */
MXFP4_API mxfp4_status mxfp4_linear_small_workspace(int64_t m, int64_t n, int64_t k, int64_t* bytes);

/* Buffer sizes of a TILED operand with `rows` rows and `k` columns (k > 0, a
 * multiple of 128; rows >= 0): *codes_bytes = 256 T * k / 2 and
 * *scales_bytes = 256 T * k / 32 with T = ceil(rows / 256).
 * Errors: INVALID_ARG for null pointers, rows < 0, or k not a positive
 *   multiple of 128. */
MXFP4_API mxfp4_status mxfp4_tiled_bytes(int64_t rows, int64_t k, int64_t* codes_bytes,
                                         int64_t* scales_bytes);

/* Host helper for the offline weight fold of a Kronecker transform: since
 * (A (x) B)^-T = A^-T (x) B^-T, quantizing the weights with KRON factors
 * (A^-T, B^-T) keeps every block dot product (T x) . (T^-T w) = x . w.
 *   m    host, n x n fp32 row-major;  out  host, n x n fp32 (written);
 *   1 <= n <= 32.  Binary64 Gauss-Jordan with partial pivoting, then
 *   transposed and rounded to fp32.
 * Errors: INVALID_ARG for null pointers or n out of range, or a singular
 *   matrix (a zero pivot). */
MXFP4_API mxfp4_status mxfp4_inverse_transpose(const float* m, int32_t n, float* out);

/* Host helper for the offline weight fold of per-channel smoothing: the
 * activations' column c is multiplied by r[c] (MXFP4_ROT_SMOOTH), so the
 * weights' column c takes 1/r[c] and every product x[c] * w[c] is kept.
 * The SmoothQuant-style scaling is the baseline "KroQuant: ..." compares its
 * transform with (abstract); the inverse scaling goes on the weights.
 *   r    host, k fp32 activation factors;  out  host, k fp32 (written):
 *        out[c] = 1/r[c], the quotient formed in binary64 and rounded once to
 *        fp32 (this equals the correctly rounded fp32 reciprocal).
 * Errors: INVALID_ARG for null pointers, k <= 0, a factor that is zero or
 *   not finite, or one whose reciprocal overflows fp32 (nothing is written
 *   past the first such factor). */
MXFP4_API mxfp4_status mxfp4_smooth_weight_factors(const float* r, int64_t k, float* out);

/* Static description of a status code (never NULL). */
MXFP4_API const char* mxfp4_status_string(int32_t status);

/* ABI version of this header (bumped on incompatible changes). */
#define MXFP4_ABI_VERSION 4
MXFP4_API int32_t mxfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
