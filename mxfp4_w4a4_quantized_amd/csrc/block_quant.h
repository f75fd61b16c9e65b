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
//  - Kronecker block transform: "KroQuant: ...", abstract and "Tiefenanalyse".
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
#pragma unroll
  for (int j = 0; j < P; ++j) {
#pragma unroll
    for (int k = 0; k < Q; ++k) {
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

// Block amax, E8M0 scale byte and packed E2M1 codes of one rotated block:
// returns the scale byte, writes the 16 code bytes (element 2j in the low
// nibble of byte j) to w.
__device__ __forceinline__ uint32_t encode_block(const float (&v)[32], uint32_t (&w)[4]) {
  // block amax (exact)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));

  // E8M0: floor(log2 amax) - 2 clamped at -127 is the biased exponent field
  // of amax minus 2 (subnormal and zero amax have field 0 and clamp).
  const uint32_t ef = __float_as_uint(amax) >> 23;
  const uint32_t sbyte = ef > 2u ? ef - 2u : 0u;
  // The block scale 2^e as fp32 (2^-127 is the subnormal 0x00400000).  The
  // converter divides by its scale operand exactly -- it equals converting
  // v * 2^-e with scale 1 for every finite input, checked on the device for
  // all bf16 values and e in [-127, 125] -- so no separate multiply is needed.
  const float scale = __uint_as_float(sbyte ? sbyte << 23 : 0x00400000u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t acc = 0;
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 0], v[8 * i + 1], scale, 0);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 2], v[8 * i + 3], scale, 1);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 4], v[8 * i + 5], scale, 2);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 6], v[8 * i + 7], scale, 3);
    w[i] = acc;
  }
  return sbyte;
}

// Rotation of one block: 0 none, 1 Hadamard-32, 2 Kronecker P x Q.
template <int ROT, int P, int Q>
__device__ __forceinline__ void rotate_block(const float* __restrict__ fa, const float* __restrict__ fb,
                                             float (&v)[32]) {
  if constexpr (ROT == 1) hadamard32(v);
  if constexpr (ROT == 2) kron32<P, Q>(fa, fb, v);
}

}  // namespace blockq
}  // namespace mxfp4
