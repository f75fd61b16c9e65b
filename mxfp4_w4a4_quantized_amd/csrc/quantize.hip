// Online MXFP4 activation quantizer for gfx950 (CDNA4).
//
// One thread owns one 32-element block: it loads the block with four 16-byte
// loads (bf16) or eight (fp32), widens to fp32, applies the optional block
// rotation entirely in registers, reduces the block amax, derives the E8M0
// scale from the amax exponent bits, converts pairs of scaled values with the
// hardware E2M1 converter (v_cvt_scalef32_pk_fp4_f32, round-to-nearest-even,
// saturating, sign kept on zero) and writes its 16 code bytes with one
// 16-byte store and its scale with one byte store.  Consecutive threads own
// consecutive blocks, so every wave writes 1 KiB of codes and 64 scale bytes
// contiguously.
//
// Method (page titles and sections as the pages give them):
//  - block format: "AMD Quark delivers MXFP4 quantization for FLUX.1-dev on
//    Instinct MI350 with 1.92x speedup", "What is MXFP4 and why does it
//    eliminate dequantization overhead?" (32-element blocks, one shared
//    scale, 4-bit elements, per the MX specification);
//  - power-of-two E8M0 scale: "Bridging the Gap Between Promise and
//    Performance for Microscaling FP4 Quantization", "Probleemstelling";
//  - Hadamard-32 micro-rotation, online and fused into quantization: same
//    page, "Methodologie: MR-GPTQ" item 1 and "GPU Kernel Ondersteuning
//    (QuTLASS)";
//  - Kronecker block transform: "KroQuant: ...", abstract and "Tiefenanalyse".
//
// Every fp32 operation below is a single IEEE operation in a fixed order (the
// library is compiled with -ffp-contract=off and the only fused operations
// are explicit fmaf calls), so codes and scales are reproducible bit for bit.
#include "internal.h"

namespace mxfp4 {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// rot: 0 none, 1 Hadamard-32, 2 Kronecker (P x Q)
template <bool BF16, int ROT, int P, int Q>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t nblk = a.rows * a.nblk_row;
  if (gid >= nblk) return;
  const uint32_t r = gid / a.nblk_row;
  const uint32_t b = gid - r * a.nblk_row;

  float v[32];
  if constexpr (BF16) {
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.x) + (int64_t)r * a.ld_x + (int64_t)b * 32);
    u32x4 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = __builtin_nontemporal_load(src + i);   // X is read once
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {q[i][0], q[i][1], q[i][2], q[i][3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_lo(w[j]);
        v[8 * i + 2 * j + 1] = bf16_hi(w[j]);
      }
    }
  } else {
    const f32x4* src = reinterpret_cast<const f32x4*>(
        static_cast<const float*>(a.x) + (int64_t)r * a.ld_x + (int64_t)b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 f = __builtin_nontemporal_load(src + i);
      v[4 * i] = f[0]; v[4 * i + 1] = f[1]; v[4 * i + 2] = f[2]; v[4 * i + 3] = f[3];
    }
  }

  if constexpr (ROT == 1) hadamard32(v);
  if constexpr (ROT == 2) kron32<P, Q>(a.fa, a.fb, v);

  // block amax (exact)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));

  // E8M0: floor(log2 amax) - 2 clamped at -127 is the biased exponent field
  // of amax minus 2 (subnormal and zero amax have field 0 and clamp).
  const uint32_t ef = __float_as_uint(amax) >> 23;
  const uint32_t sbyte = ef > 2u ? ef - 2u : 0u;
  // 2^-e as an fp32 with exponent field 254 - sbyte (always normal)
  const float inv = __uint_as_float((254u - sbyte) << 23);

  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t acc = 0;
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 0] * inv, v[8 * i + 1] * inv, 1.0f, 0);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 2] * inv, v[8 * i + 3] * inv, 1.0f, 1);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 4] * inv, v[8 * i + 5] * inv, 1.0f, 2);
    acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, v[8 * i + 6] * inv, v[8 * i + 7] * inv, 1.0f, 3);
    w[i] = acc;
  }
  uint4* dst = reinterpret_cast<uint4*>(a.codes) + gid;
  *dst = make_uint4(w[0], w[1], w[2], w[3]);   // the GEMM reads these next: keep them cached
  a.scales[gid] = static_cast<uint8_t>(sbyte);
}

template <bool BF16>
hipError_t dispatch(const QuantArgs& a, hipStream_t s) {
  const uint32_t nblk = a.rows * a.nblk_row;
  const dim3 grid((nblk + kThreads - 1) / kThreads), block(kThreads);
  if (a.rot == 0) {
    quantize_kernel<BF16, 0, 1, 32><<<grid, block, 0, s>>>(a);
  } else if (a.rot == 1) {
    quantize_kernel<BF16, 1, 1, 32><<<grid, block, 0, s>>>(a);
  } else {
    switch (a.p) {
      case 1: quantize_kernel<BF16, 2, 1, 32><<<grid, block, 0, s>>>(a); break;
      case 2: quantize_kernel<BF16, 2, 2, 16><<<grid, block, 0, s>>>(a); break;
      case 4: quantize_kernel<BF16, 2, 4, 8><<<grid, block, 0, s>>>(a); break;
      case 8: quantize_kernel<BF16, 2, 8, 4><<<grid, block, 0, s>>>(a); break;
      case 16: quantize_kernel<BF16, 2, 16, 2><<<grid, block, 0, s>>>(a); break;
      case 32: quantize_kernel<BF16, 2, 32, 1><<<grid, block, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, bool bf16, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  return bf16 ? dispatch<true>(a, s) : dispatch<false>(a, s);
}

}  // namespace mxfp4
