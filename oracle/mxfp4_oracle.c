/*
 * Plain CPU oracle for the W4A4 MXFP4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the GPU path must compute;
 * only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code, header, table or constant with
 * the HIP library, and it includes nothing from it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (see oracle/build.py).  All
 * float arithmetic below is IEEE binary32/binary64 with round-to-nearest-even,
 * no contraction: every fused multiply-add is an explicit fmaf().
 *
 * Sources (page titles and sections as the pages give them):
 *  [P2]  "AMD Quark delivers MXFP4 quantization for FLUX.1-dev on Instinct MI350
 *        with 1.92x speedup", section "What is MXFP4 and why does it eliminate
 *        dequantization overhead?" -- 4-bit elements, blocks of 32 sharing one
 *        scale, defined by the Microscaling (MX) specification.
 *  [P3m] "Bridging the Gap Between Promise and Performance for Microscaling FP4
 *        Quantization", Technische samenvatting, "Probleemstelling" -- MXFP4
 *        uses group size 32 and power-of-two E8M0 scales;
 *        "Methodologie: MR-GPTQ", item 1 -- block-wise Hadamard rotation of
 *        weights and activations before quantizing.
 *  [P3k] same page, "GPU Kernel Ondersteuning (QuTLASS)" -- the rotation runs
 *        online, fused into the quantization and matmul kernels.
 *  [P4]  "KroQuant: Effiziente Post-Training-Quantisierung fuer Diffusion
 *        Transformers mittels Kronecker-Produkt-Struktur", abstract and
 *        "Tiefenanalyse" -- a learned Kronecker-structured invertible transform
 *        on each 32-element activation block; "Hintergrund" -- the inverse goes
 *        on the weights.
 *  [P4s] same page, the comparison with SmoothQuant (per-channel scaling of the
 *        activations, with the inverse scaling folded into the weights).
 *  [P3f] "Bridging the Gap ...", "Methodologie: MR-GPTQ", item 2 -- for MXFP4
 *        the exponent of the block scale is re-fitted ("scale fitting") to
 *        match the grid to the data and lower the quantization error.
 *  [MX]  the OCP Microscaling Formats (MX) v1.0 specification that [P2] names:
 *        FP4 E2M1 element (bias 1, one mantissa bit, no Inf/NaN), E8M0 scale
 *        (value 2^(byte-127)), shared exponent floor(log2(amax)) - emax_elem
 *        with emax_elem = 2 for E2M1.
 *
 * Readings taken where the pages are silent are marked READING.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>

/* ------------------------------------------------------------------------- */
/* Element and scale formats                                                  */
/* ------------------------------------------------------------------------- */

/* E2M1 magnitudes in code order 0..7 ([MX] FP4 E2M1; [P2] 4 bits/element). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Q1: value of a 4-bit E2M1 code; bit 3 is the sign. */
double oracle_e2m1_value(int code)
{
    double m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* Value of an E8M0 scale byte: 2^(byte-127).  byte 255 (NaN in [MX]) is
 * never produced for finite data and is returned as NaN here. */
double oracle_e8m0_value(int byte)
{
    if (byte == 255) return NAN;
    return ldexp(1.0, byte - 127);
}

/* floor(log2(a)) for finite a > 0, exact: frexpf gives a = m * 2^ex with
 * m in [0.5, 1), so floor(log2 a) = ex - 1 (subnormals included). */
static int floor_log2f(float a)
{
    int ex;
    (void)frexpf(a, &ex);
    return ex - 1;
}

/* Q2: shared block exponent ([MX]; [P3m] Probleemstelling: power-of-two E8M0).
 *   e = floor(log2(amax)) - 2, clamped below at -127; byte = e + 127.
 * READING: amax == 0 gives byte 0 (e = -127); the lower clamp only acts for
 * amax < 2^-125.  No upper clamp is needed for finite amax (e <= 125). */
int oracle_e8m0_from_amax(float amax)
{
    int e;
    if (amax == 0.0f) return 0;
    e = floor_log2f(amax) - 2;
    if (e < -127) e = -127;
    return e + 127;
}

/* Q3 magnitude index for a scaled magnitude t >= 0: round to the nearest E2M1
 * magnitude, ties to the code with the even mantissa bit (even index), values
 * beyond the largest magnitude saturate to it (6).  Distances are taken in
 * binary64, where t - g is exact for every fp32 t near a midpoint. */
int oracle_e2m1_index(float t)
{
    int best = 0, i;
    double bd;
    if (t >= 6.0f) return 7;     /* saturation (also keeps distances exact) */
    bd = fabs((double)t - E2M1_MAG[0]);
    for (i = 1; i < 8; ++i) {
        double d = fabs((double)t - E2M1_MAG[i]);
        if (d < bd || (d == bd && (i & 1) == 0 && (best & 1) == 1)) {
            best = i;
            bd = d;
        }
    }
    return best;
}

/* Q3: 4-bit code of y in a block with shared exponent e.
 * t = |y| * 2^-e is formed with ldexpf (exact whenever t is normal, which is
 * the case for every t that can round to a non-zero magnitude).
 * READING: the sign bit is copied from y even when the magnitude rounds to 0
 * (IEEE-style signed zero), so -0.0 and tiny negatives give code 0x8. */
int oracle_e2m1_encode(float y, int e)
{
    float t = ldexpf(fabsf(y), -e);
    int code = oracle_e2m1_index(t);
    if (signbit(y)) code |= 8;
    return code;
}

/* ------------------------------------------------------------------------- */
/* Block rotations                                                            */
/* ------------------------------------------------------------------------- */

/* Q5: normalized Hadamard-32 ([P3m] Methodologie item 1; [P3k]).
 * H[i][j] = (-1)^popcount(i & j) / sqrt(32) (Sylvester order).
 * READING (op order, so that fp32 results are reproducible): fast
 * Walsh-Hadamard butterflies with strides 1, 2, 4, 8, 16 in that order, each
 * pair (u, v) -> (u + v, u - v) rounded to fp32, then one fp32 multiply of
 * every element by c = fp32(1/sqrt(32)).  No fused operations. */
void oracle_fwht32(const float* x, float* y)
{
    float v[32];
    int h, i, j;
    const float c = (float)(1.0 / sqrt(32.0));
    memcpy(v, x, sizeof v);
    for (h = 1; h < 32; h <<= 1) {
        for (i = 0; i < 32; i += 2 * h) {
            for (j = i; j < i + h; ++j) {
                float u = v[j], w = v[j + h];
                v[j] = u + w;
                v[j + h] = u - w;
            }
        }
    }
    for (i = 0; i < 32; ++i) y[i] = v[i] * c;
}

/* Q6: Kronecker block transform y = (A (x) B) x ([P4] abstract, Tiefenanalyse).
 * A is p x p, B is q x q, both row-major fp32, p*q = 32.  With the block seen
 * as the p x q matrix Xm[j][l] = x[q*j + l], y = vec(A * Xm * B^T), i.e.
 * y[q*i + k] = sum_j A[i][j] * sum_l B[k][l] * Xm[j][l].
 * READING (op order): stage 1 forms U[j][k] as a chain over l ascending,
 * stage 2 forms Y[i][k] as a chain over j ascending; a chain starts with the
 * rounded first product and continues with fmaf(coef, value, acc). */
void oracle_kron_apply(const float* A, int p, const float* B, int q,
                       const float* x, float* y)
{
    float U[32];
    int i, j, k, l;
    for (j = 0; j < p; ++j) {
        for (k = 0; k < q; ++k) {
            float acc = B[k * q + 0] * x[q * j + 0];
            for (l = 1; l < q; ++l) acc = fmaf(B[k * q + l], x[q * j + l], acc);
            U[j * q + k] = acc;
        }
    }
    for (i = 0; i < p; ++i) {
        for (k = 0; k < q; ++k) {
            float acc = A[i * p + 0] * U[0 * q + k];
            for (j = 1; j < p; ++j) acc = fmaf(A[i * p + j], U[j * q + k], acc);
            y[q * i + k] = acc;
        }
    }
}

/* Inverse-transpose of an n x n fp32 matrix, for folding the inverse of the
 * activation transform into the weights ([P4] Hintergrund: transform on the
 * activations, its inverse on the weights).  Since (A (x) B)^-T =
 * A^-T (x) B^-T, the weight side of a Kronecker transform is again a
 * Kronecker transform with these factors.  Computed in binary64 by
 * Gauss-Jordan elimination with partial pivoting on [M | I], then transposed
 * and rounded to fp32.  Returns 0 on success, -1 if a pivot is zero. */
int oracle_inverse_transpose(const float* m, int n, float* out)
{
    double a[32][64];
    int r, c, k, piv;
    if (n < 1 || n > 32) return -1;
    for (r = 0; r < n; ++r) {
        for (c = 0; c < n; ++c) a[r][c] = (double)m[r * n + c];
        for (c = 0; c < n; ++c) a[r][n + c] = (r == c) ? 1.0 : 0.0;
    }
    for (k = 0; k < n; ++k) {
        double best = fabs(a[k][k]);
        piv = k;
        for (r = k + 1; r < n; ++r)
            if (fabs(a[r][k]) > best) { best = fabs(a[r][k]); piv = r; }
        if (best == 0.0) return -1;
        if (piv != k)
            for (c = 0; c < 2 * n; ++c) { double t = a[k][c]; a[k][c] = a[piv][c]; a[piv][c] = t; }
        {
            double d = a[k][k];
            for (c = 0; c < 2 * n; ++c) a[k][c] /= d;
        }
        for (r = 0; r < n; ++r) {
            double f;
            if (r == k) continue;
            f = a[r][k];
            if (f == 0.0) continue;
            for (c = 0; c < 2 * n; ++c) a[r][c] -= f * a[k][c];
        }
    }
    for (r = 0; r < n; ++r)
        for (c = 0; c < n; ++c) out[r * n + c] = (float)a[c][n + r];
    return 0;
}

/* Weight side of per-channel smoothing ([P4s]: the activations are divided
 * by the smoothing factor s[c], the weights multiplied by it).  With the
 * activation factor r[c] = 1/s[c] (the multiplier the quantizer applies),
 * the weight factor is 1/r[c]: the quotient is formed in binary64 and
 * rounded to fp32.  Binary64 has more than 2*24 + 2 bits, so this double
 * rounding of a quotient of two fp32 values gives the correctly rounded fp32
 * reciprocal.  Returns 0, or -1 if some r[c] is zero or not finite, or its
 * reciprocal is not a finite fp32 (k < 0 is an error too). */
int oracle_smooth_weight_factors(const float* r, int64_t k, float* out)
{
    int64_t c;
    if (k < 0) return -1;
    for (c = 0; c < k; ++c) {
        double q;
        float f;
        if (!isfinite(r[c]) || r[c] == 0.0f) return -1;
        q = 1.0 / (double)r[c];
        f = (float)q;
        if (!isfinite(f)) return -1;
        out[c] = f;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Quantizer                                                                   */
/* ------------------------------------------------------------------------- */

enum { ROT_NONE = 0, ROT_H32 = 1, ROT_KRON = 2, ROT_SMOOTH = 3 };

/* bf16 -> fp32 widening is exact: the bf16 bits are the upper half. */
static float widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Sum of squared errors of one block encoded with shared exponent e, in
 * binary64: the sum runs over the elements in order, each term the exact
 * difference v - x_hat squared (every step a single binary64 operation).
 * READING ([P3f] names scale fitting without a formula): the fitted exponent
 * is the one of e0 - 1, e0, e0 + 1 (e0 the rule of Q2) with the smallest
 * such error; a candidate replaces the current best only when strictly
 * smaller, tried in the order e0, e0 + 1, e0 - 1, so ties keep e0.  e0 - 1 is
 * not tried at the lower clamp (e0 = -127); e0 + 1 <= 126 always holds for
 * finite blocks. */
static double block_sse(const float* v, int e)
{
    double s = 0.0;
    int i;
    for (i = 0; i < 32; ++i) {
        int c = oracle_e2m1_encode(v[i], e);
        double xh = oracle_e2m1_value(c) * ldexp(1.0, e);
        double d = (double)v[i] - xh;
        double d2 = d * d;
        s = s + d2;
    }
    return s;
}

/* One 32-element block: optional rotation, block amax, E8M0 scale (the Q2
 * rule, or the fitted exponent when fit != 0), E2M1 codes packed two per
 * byte.  For ROT_SMOOTH, A points at this block's 32 per-channel factors.
 * READING (nibble order): element 2j goes to the low nibble of byte j and
 * element 2j+1 to the high nibble.
 * READING ([P4s]): the smoothing division by the per-channel factor s is one
 * IEEE fp32 multiply by the caller's factor r = 1/s. */
static void quantize_block(const float* xin, int rot, const float* A, int p,
                           const float* B, int q, int fit, uint8_t* codes16,
                           uint8_t* scale)
{
    float v[32];
    float amax = 0.0f;
    int i, byte, e;
    if (rot == ROT_H32) oracle_fwht32(xin, v);
    else if (rot == ROT_KRON) oracle_kron_apply(A, p, B, q, xin, v);
    else if (rot == ROT_SMOOTH) {
        for (i = 0; i < 32; ++i) v[i] = xin[i] * A[i];
    } else memcpy(v, xin, sizeof v);
    for (i = 0; i < 32; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    byte = oracle_e8m0_from_amax(amax);
    e = byte - 127;
    if (fit) {
        double best = block_sse(v, e), err;
        int e0 = e;
        err = block_sse(v, e0 + 1);
        if (err < best) { best = err; e = e0 + 1; }
        if (e0 > -127) {
            err = block_sse(v, e0 - 1);
            if (err < best) { best = err; e = e0 - 1; }
        }
        byte = e + 127;
    }
    for (i = 0; i < 16; ++i) {
        int lo = oracle_e2m1_encode(v[2 * i], e);
        int hi = oracle_e2m1_encode(v[2 * i + 1], e);
        codes16[i] = (uint8_t)(lo | (hi << 4));
    }
    *scale = (uint8_t)byte;
}

static int check_args(int64_t rows, int64_t k, int64_t ld, int rot, int p, int q)
{
    if (rows < 0 || k < 0 || (k % 32) != 0 || ld < k) return -1;
    if (rot == ROT_KRON && (p < 1 || q < 1 || p * q != 32)) return -1;
    if (rot < ROT_NONE || rot > ROT_SMOOTH) return -1;
    return 0;
}

/* Quantize a row-major fp32 matrix x[rows][ld] (first k columns).
 * codes: rows x k/2 bytes, scales: rows x k/32 bytes, both dense row-major.
 * ROT_SMOOTH: A holds k per-channel factors.  fit != 0: fitted exponents. */
int oracle_quantize_f32_ex(const float* x, int64_t rows, int64_t k, int64_t ld,
                           int rot, const float* A, int p, const float* B, int q,
                           int fit, uint8_t* codes, uint8_t* scales)
{
    int64_t r, b, nb = k / 32;
    if (check_args(rows, k, ld, rot, p, q)) return -1;
    for (r = 0; r < rows; ++r)
        for (b = 0; b < nb; ++b)
            quantize_block(x + r * ld + 32 * b, rot,
                           rot == ROT_SMOOTH ? A + 32 * b : A, p, B, q, fit,
                           codes + r * (k / 2) + 16 * b, scales + r * nb + b);
    return 0;
}

/* Same for bf16 input (raw uint16 bit patterns), widened exactly to fp32. */
int oracle_quantize_bf16_ex(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                            int rot, const float* A, int p, const float* B, int q,
                            int fit, uint8_t* codes, uint8_t* scales)
{
    int64_t r, b, nb = k / 32;
    float blk[32];
    int i;
    if (check_args(rows, k, ld, rot, p, q)) return -1;
    for (r = 0; r < rows; ++r)
        for (b = 0; b < nb; ++b) {
            for (i = 0; i < 32; ++i) blk[i] = widen_bf16(x[r * ld + 32 * b + i]);
            quantize_block(blk, rot, rot == ROT_SMOOTH ? A + 32 * b : A, p, B, q, fit,
                           codes + r * (k / 2) + 16 * b, scales + r * nb + b);
        }
    return 0;
}

int oracle_quantize_f32(const float* x, int64_t rows, int64_t k, int64_t ld,
                        int rot, const float* A, int p, const float* B, int q,
                        uint8_t* codes, uint8_t* scales)
{
    return oracle_quantize_f32_ex(x, rows, k, ld, rot, A, p, B, q, 0, codes, scales);
}

int oracle_quantize_bf16(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                         int rot, const float* A, int p, const float* B, int q,
                         uint8_t* codes, uint8_t* scales)
{
    return oracle_quantize_bf16_ex(x, rows, k, ld, rot, A, p, B, q, 0, codes, scales);
}

/* Rotation only (no quantization), for checking the rotation stage alone. */
int oracle_rotate_f32(const float* x, int64_t rows, int64_t k, int rot,
                      const float* A, int p, const float* B, int q, float* y)
{
    int64_t r, b;
    if (check_args(rows, k, k, rot, p, q)) return -1;
    for (r = 0; r < rows; ++r)
        for (b = 0; b < k / 32; ++b) {
            const float* s = x + r * k + 32 * b;
            float* d = y + r * k + 32 * b;
            if (rot == ROT_H32) oracle_fwht32(s, d);
            else if (rot == ROT_KRON) oracle_kron_apply(A, p, B, q, s, d);
            else if (rot == ROT_SMOOTH) {
                int i;
                for (i = 0; i < 32; ++i) d[i] = s[i] * A[32 * b + i];
            } else memcpy(d, s, 32 * sizeof(float));
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Dequantize and GEMM                                                         */
/* ------------------------------------------------------------------------- */

/* x_hat[r][c] = e2m1(code) * 2^(scale - 127), in binary64 (exact). */
void oracle_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                       int64_t k, double* out)
{
    int64_t r, c, nb = k / 32;
    for (r = 0; r < rows; ++r)
        for (c = 0; c < k; ++c) {
            uint8_t byte = codes[r * (k / 2) + c / 2];
            int code = (c & 1) ? (byte >> 4) : (byte & 15);
            out[r * k + c] = oracle_e2m1_value(code) *
                             oracle_e8m0_value(scales[r * nb + c / 32]);
        }
}

/* Q7 at chosen entries: Y[m][n] = sum_k a_hat[m][k] * b_hat[n][k] in binary64,
 * for `count` index pairs (mi[t], ni[t]).  Each product is exact in binary64;
 * the sum is taken in ascending k.  ([P2] "MXFP4 quantization for diffusion
 * models": the GEMM takes MXFP4 operands directly; Y = A * B^T.) */
void oracle_gemm_entries(const uint8_t* a_codes, const uint8_t* a_scales,
                         const uint8_t* b_codes, const uint8_t* b_scales,
                         int64_t k, const int64_t* mi, const int64_t* ni,
                         int64_t count, double* out)
{
    int64_t t, c, nb = k / 32;
    for (t = 0; t < count; ++t) {
        const uint8_t* ac = a_codes + mi[t] * (k / 2);
        const uint8_t* bc = b_codes + ni[t] * (k / 2);
        const uint8_t* as = a_scales + mi[t] * nb;
        const uint8_t* bs = b_scales + ni[t] * nb;
        double acc = 0.0;
        for (c = 0; c < k; ++c) {
            int ca = (c & 1) ? (ac[c / 2] >> 4) : (ac[c / 2] & 15);
            int cb = (c & 1) ? (bc[c / 2] >> 4) : (bc[c / 2] & 15);
            double xa = oracle_e2m1_value(ca) * oracle_e8m0_value(as[c / 32]);
            double xb = oracle_e2m1_value(cb) * oracle_e8m0_value(bs[c / 32]);
            acc += xa * xb;
        }
        out[t] = acc;
    }
}

/* ------------------------------------------------------------------------- */
/* Array forms of the scalar rules, for exhaustive checks from Python.        */
/* ------------------------------------------------------------------------- */

void oracle_e2m1_index_array(const float* t, int64_t n, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_index(t[i]);
}

void oracle_e2m1_encode_array(const float* y, int64_t n, int e, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_encode(y[i], e);
}

void oracle_e8m0_from_amax_array(const float* a, int64_t n, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e8m0_from_amax(a[i]);
}
