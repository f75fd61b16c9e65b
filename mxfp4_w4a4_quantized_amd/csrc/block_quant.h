// Per-block MXFP4 quantization arithmetic shared by the quantizer kernel and
// the fused small-M linear kernel, so both produce the same codes and scales
// bit for bit: widening, the optional block rotation, the block amax, the
// E8M0 scale and the E2M1 encoding.
//
// Method (page titles and sections as the pages give them):
//  - block format: "AMD Quark delivers MXFP4 quantization for FLUX.1-dev on
//    Instinct MI350 with 1.92x speedup", "What is MXFP4 and why does it
//    eliminate dequantization overhead?" (32-element blocks, one shared
//    scale, 4-bit elements, per the MX specification);
//  - power-of-two E8M0 scale: "Bridging the Gap Between Promise and
//    Performance for Microscaling FP4 Quantization", "Probleemstelling";
//  - Hadamard-32 micro-rotation: same page, "Methodologie: MR-GPTQ" item 1;
//  - Kronecker block transform: "KroQuant: ...", abstract and "Tiefenanalyse";
//  - per-channel smoothing, the SmoothQuant baseline that page compares with:
//    one fp32 multiply by the caller's per-channel factor;
//  - scale fitting: "Bridging the Gap ...", "Methodologie: MR-GPTQ" item 2
//    (the exponent of the block scale re-fitted to the data; the rule used
//    here: the exponent among e0 - 1, e0, e0 + 1 with the smallest squared
//    error, each error summed in binary64 in element order, ties keep e0,
//    then e0 + 1).
//
// Every fp32 operation is a single IEEE operation in a fixed order (the
// library is compiled with -ffp-contract=off and the only fused operations
// are explicit fmaf calls), so results are reproducible bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mxfp4 {
namespace blockq {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Normalized Hadamard-32 (Sylvester order) as five butterfly stages with
// strides 1, 2, 4, 8, 16, then one multiply by fp32(1/sqrt(32)).
__device__ __forceinline__ void hadamard32(float (&v)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float u = v[j], w = v[j + h];
        v[j] = u + w;
        v[j + h] = u - w;
      }
    }
  }
  const float c = __uint_as_float(0x3E3504F3u);  // nearest fp32 to 1/sqrt(32)
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = v[i] * c;
}

// y = (A (x) B) x on the block seen as the P x Q matrix Xm[j][l] = x[Q*j+l]:
// stage 1 U[j][k] = chain_l B[k][l] Xm[j][l], stage 2 y[Q*i+k] =
// chain_j A[i][j] U[j][k]; each chain is the rounded first product followed
// by fused multiply-adds in ascending order.  The factor loads are uniform
// across the wave and become scalar loads.
template <int P, int Q>
__device__ __forceinline__ void kron32(const float* __restrict__ fa, const float* __restrict__ fb,
                                       float (&v)[32]) {
  static_assert(P * Q == 32, "P*Q must be 32");
  float u[32];
  // row k of B is used by all P chains of stage 1 at once (fewer factor
  // registers live at a time than going block row by block row)
#pragma unroll
  for (int k = 0; k < Q; ++k) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      float acc = fb[k * Q] * v[Q * j];
#pragma unroll
      for (int l = 1; l < Q; ++l) acc = __builtin_fmaf(fb[k * Q + l], v[Q * j + l], acc);
      u[j * Q + k] = acc;
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
#pragma unroll
    for (int k = 0; k < Q; ++k) {
      float acc = fa[i * P] * u[k];
#pragma unroll
      for (int j = 1; j < P; ++j) acc = __builtin_fmaf(fa[i * P + j], u[j * Q + k], acc);
      v[Q * i + k] = acc;
    }
  }
}

// E8M0 byte of the block rule: floor(log2 amax) - 2 clamped at -127 is the
// biased exponent field of amax minus 2 (subnormal and zero amax have field 0
// and clamp).
__device__ __forceinline__ uint32_t sbyte_of_amax(float amax) {
  const uint32_t ef = __float_as_uint(amax) >> 23;
  return ef > 2u ? ef - 2u : 0u;
}

__device__ __forceinline__ uint32_t rule_sbyte(const float (&v)[32]) {
  float amax = 0.0f;   // exact
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  return sbyte_of_amax(amax);
}

// The block scale 2^(sbyte - 127) as fp32 (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float scale_of(uint32_t sbyte) {
  return __uint_as_float(sbyte ? sbyte << 23 : 0x00400000u);
}

// Packed E2M1 codes (element 2j in the low nibble of byte j) of the block at
// scale byte sbyte.  The converter divides by its scale operand exactly -- it
// equals converting v * 2^-e with scale 1 for every finite input, checked on
// the device for all bf16 values and e in [-127, 125] -- then rounds to
// nearest even and saturates, keeping the sign of values that round to zero.
__device__ __forceinline__ void encode_at(const float (&v)[32], uint32_t sbyte, uint32_t (&w)[4]) {
  const float scale = scale_of(sbyte);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t acc = 0;
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 0], v[8 * i + 1], scale, 0);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 2], v[8 * i + 3], scale, 1);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 4], v[8 * i + 5], scale, 2);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 6], v[8 * i + 7], scale, 3);
    w[i] = acc;
  }
}

// Block amax, E8M0 scale byte and packed E2M1 codes of one rotated block:
// returns the scale byte, writes the 16 code bytes to w.
__device__ __forceinline__ uint32_t encode_block(const float (&v)[32], uint32_t (&w)[4]) {
  const uint32_t sbyte = rule_sbyte(v);
  encode_at(v, sbyte, w);
  return sbyte;
}

// Block amax, E8M0 byte and codes of an untransformed bf16 block, straight
// from its 16 packed dwords (element 2j in the low half of dword j).  For
// finite bf16 values the magnitude bits order like the magnitudes, so the
// block amax is a packed 16-bit unsigned max over the bits with the sign
// cleared, and its biased exponent is those bits >> 7 -- the fp32 exponent
// field of the same value.  The converter then reads the bf16 pairs directly
// (widening bf16 to fp32 is exact, so this is the f32 conversion of the
// widened values).  Same bytes as widening, encode_block and the f32
// converter, with neither the widening nor a float max per element.
__device__ __forceinline__ uint32_t encode_block_bf16(const uint32_t (&d)[16], uint32_t (&w)[4]) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = __builtin_bit_cast(u16x2, d[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 16; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[i] & 0x7FFF7FFFu));
  const uint32_t ef = (uint32_t)(m[0] > m[1] ? m[0] : m[1]) >> 7;
  const uint32_t sbyte = ef > 2u ? ef - 2u : 0u;
  const float scale = scale_of(sbyte);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t acc = 0;
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, __builtin_bit_cast(bf16x2, d[4 * i + 0]), scale, 0);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, __builtin_bit_cast(bf16x2, d[4 * i + 1]), scale, 1);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, __builtin_bit_cast(bf16x2, d[4 * i + 2]), scale, 2);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(acc, __builtin_bit_cast(bf16x2, d[4 * i + 3]), scale, 3);
    w[i] = acc;
  }
  return sbyte;
}

// Value of a 4-bit E2M1 code (bit 3 the sign).
__device__ __forceinline__ double e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const double mag = m < 4u ? 0.5 * (double)m : (m == 4u ? 2.0 : (m == 5u ? 3.0 : (m == 6u ? 4.0 : 6.0)));
  return (c & 8u) ? -mag : mag;
}

// Squared error of the block encoded at scale byte sbyte, in binary64: over
// the elements in order, d = v - x_hat (x_hat = code value * scale, exact),
// s = s + d * d, each a single binary64 operation.
__device__ __forceinline__ double block_sse(const float (&v)[32], uint32_t sbyte) {
  uint32_t w[4];
  encode_at(v, sbyte, w);
  const double sc = (double)scale_of(sbyte);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = (w[i >> 3] >> (4 * (i & 7))) & 0xFu;
    const double xh = e2m1_value(c) * sc;
    const double d = (double)v[i] - xh;
    const double d2 = d * d;
    s = s + d2;
  }
  return s;
}

// Scale-fitted encoding of one block (see the header comment for the rule).
__device__ __forceinline__ uint32_t encode_block_fit(const float (&v)[32], uint32_t (&w)[4]) {
  const uint32_t s0 = rule_sbyte(v);
  uint32_t best = s0;
  double err = block_sse(v, s0);
  const double e_up = block_sse(v, s0 + 1u);
  if (e_up < err) {
    err = e_up;
    best = s0 + 1u;
  }
  if (s0 > 0u) {
    const double e_dn = block_sse(v, s0 - 1u);
    if (e_dn < err) best = s0 - 1u;
  }
  encode_at(v, best, w);
  return best;
}

template <bool FIT>
__device__ __forceinline__ uint32_t encode_block_sel(const float (&v)[32], uint32_t (&w)[4]) {
  if constexpr (FIT) return encode_block_fit(v, w);
  else return encode_block(v, w);
}

// Transform of one block: 0 none, 1 Hadamard-32, 2 Kronecker P x Q (factors
// fa, fb), 3 per-channel smoothing (fa = this block's 32 factors).
template <int ROT, int P, int Q>
__device__ __forceinline__ void rotate_block(const float* __restrict__ fa, const float* __restrict__ fb,
                                             float (&v)[32]) {
  if constexpr (ROT == 1) hadamard32(v);
  if constexpr (ROT == 2) kron32<P, Q>(fa, fb, v);
  if constexpr (ROT == 3) {
    typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f4 r = *reinterpret_cast<const f4*>(fa + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = v[4 * i + j] * r[j];
    }
  }
}

}  // namespace blockq
}  // namespace mxfp4
