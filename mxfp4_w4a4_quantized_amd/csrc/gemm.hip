// MXFP4 x MXFP4 GEMM for gfx950 on the block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 (both operands E2M1, cbsz = blgp = 4).
//
// Y[m][n] = sum_k a_hat[m][k] * b_hat[n][k]; A (activations) and B (weights)
// are both K-major packed E2M1 with one E8M0 byte per 32-element block.  The
// kernel reads the packed codes and scale bytes directly -- there is no
// dequantize pass -- accumulates in fp32 and writes fp32 or bf16 ("AMD Quark
// delivers MXFP4 quantization for FLUX.1-dev on Instinct MI350 with 1.92x
// speedup", sections "MXFP4 quantization for diffusion models" and "What is
// MXFP4 and why does it eliminate dequantization overhead?").
//
// Operand layout of the MFMA with FP4 operands (checked on the device): lane l
// supplies row (l % 16) of its operand and the 32 consecutive K elements
// 32*(l/16) .. +31 as 16 packed bytes (low nibble first) -- exactly 16
// consecutive bytes of a K-major packed row -- plus one scale byte (selected
// by op_sel from a 32-bit register) that scales those 32 elements, i.e. one
// MX block.  The result lane l holds D[4*(l/16) + r][l % 16], r = 0..3.
//
// Design:
//  * The weight tile feeds the MFMA's first operand and the activation tile
//    its second, so D = W_tile * X_tile^T and each lane ends with four
//    consecutive output columns of one output row: 16-byte fp32 / 8-byte bf16
//    stores.
//  * A pipeline stage covers 256 K elements = 128 code bytes + 8 scale bytes
//    per row.  Within a stage, lane group g = l/16 always owns the adjacent
//    blocks 2g and 2g+1: the two MFMAs of the stage (sub-steps j = 0, 1) take
//    block 2g+j from lane group g.  A lane thus reads 32 contiguous code
//    bytes and one 16-bit pair of scale bytes per operand fragment, and the
//    scale byte for sub-step j is simply op_sel = j.  Any assignment of blocks
//    to (sub-step, lane group) gives the same sum as long as both operands use
//    the same one.
//  * Codes and scales are staged through LDS, double-buffered, one barrier
//    per stage; 16-byte chunks are XOR-swizzled by (row & 7) so the 16-row
//    fragment reads hit distinct banks.
//  * Rows beyond M or N are clamped to a valid row (their results are never
//    stored); blocks beyond K are zero-filled, codes and scales alike, so a
//    K tail contributes exactly 0.
#include "internal.h"

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int KS = 256;        // K elements per pipeline stage
constexpr int KSB = KS / 2;    // code bytes per row per stage
constexpr int CPR = KSB / 16;  // 16-byte chunks per row per stage
constexpr int SPR = KS / 32;   // scale bytes per row per stage

template <int J>
__device__ __forceinline__ v4f mma_fp4(const uint4& a, const uint4& b, const v4f& c, int sa, int sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, J, sa, J, sb);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int TN, int TM, int WN, int WM, bool BF16OUT>
__global__ __launch_bounds__((TN / WN) * (TM / WM) * 64) void gemm_kernel(GemmArgs g, int y_vec,
                                                                           int s_vec) {
  constexpr int NWN = TN / WN, NWM = TM / WM, NT = NWN * NWM * 64;
  constexpr int FN = WN / 16, FM = WM / 16;
  constexpr int ROWS = TN + TM;
  constexpr int CHUNKS = ROWS * CPR;
  constexpr int CPT = CHUNKS / NT;
  constexpr int SROWS = (ROWS + NT - 1) / NT;  // scale rows per thread
  static_assert(CHUNKS % NT == 0, "tile rows must split evenly over threads");

  __shared__ __attribute__((aligned(16))) uint8_t sc[2][ROWS * KSB];
  __shared__ __attribute__((aligned(16))) uint8_t ss[2][ROWS * SPR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % NWN, wm = wave / NWN;
  const int tiles_n = (g.n + TN - 1) / TN;
  const int tile_n = blockIdx.x % tiles_n, tile_m = blockIdx.x / tiles_n;
  const int n0 = tile_n * TN, m0 = tile_m * TM;
  const int kbytes = g.k / 2;
  const int kblocks = g.k / 32;
  const int nk = (g.k + KS - 1) / KS;

  // ---- global -> register staging plan (fixed for the whole K loop)
  const uint8_t* csrc[CPT];
  int cchunk[CPT], coff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * NT;
    const int row = c / CPR, ch = c % CPR;
    const uint8_t* base;
    if (row < TN) {
      const int gr = min(n0 + row, g.n - 1);
      base = g.b_codes + (int64_t)gr * kbytes;
    } else {
      const int gr = min(m0 + row - TN, g.m - 1);
      base = g.a_codes + (int64_t)gr * kbytes;
    }
    csrc[i] = base + ch * 16;
    cchunk[i] = ch;
    coff[i] = row * KSB + ((ch ^ (row & 7)) << 4);
  }
  const uint8_t* ssrc[SROWS];
  bool sown[SROWS];
#pragma unroll
  for (int i = 0; i < SROWS; ++i) {
    const int row = tid + i * NT;
    sown[i] = row < ROWS;
    const int r = sown[i] ? row : 0;
    if (r < TN) ssrc[i] = g.b_scales + (int64_t)min(n0 + r, g.n - 1) * kblocks;
    else ssrc[i] = g.a_scales + (int64_t)min(m0 + r - TN, g.m - 1) * kblocks;
  }

  uint4 creg[CPT];
  uint2 sreg[SROWS];
  auto load_stage = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const bool ok = kt * CPR + cchunk[i] < kblocks;  // chunk = one 32-block
      creg[i] = ok ? *reinterpret_cast<const uint4*>(csrc[i] + kt * KSB) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SROWS; ++i) {
      if (!sown[i]) continue;
      const int b0 = kt * SPR;
      if (s_vec && b0 + SPR <= kblocks) {
        sreg[i] = *reinterpret_cast<const uint2*>(ssrc[i] + b0);
      } else {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (b0 + t < kblocks) lo |= (uint32_t)ssrc[i][b0 + t] << (8 * t);
          if (b0 + 4 + t < kblocks) hi |= (uint32_t)ssrc[i][b0 + 4 + t] << (8 * t);
        }
        sreg[i] = make_uint2(lo, hi);
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(&sc[buf][coff[i]]) = creg[i];
#pragma unroll
    for (int i = 0; i < SROWS; ++i)
      if (sown[i]) *reinterpret_cast<uint2*>(&ss[buf][(tid + i * NT) * SPR]) = sreg[i];
  };

  v4f acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lg = lane >> 4;

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);

    int sw[FN], sx[FM];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int row = wn * WN + f * 16 + lr;
      sw[f] = *reinterpret_cast<const uint16_t*>(&ss[buf][row * SPR + 2 * lg]);
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int row = TN + wm * WM + f * 16 + lr;
      sx[f] = *reinterpret_cast<const uint16_t*>(&ss[buf][row * SPR + 2 * lg]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 wf[FN], xf[FM];
      const int ch = 2 * lg + j;
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int row = wn * WN + f * 16 + lr;
        wf[f] = *reinterpret_cast<const uint4*>(&sc[buf][row * KSB + ((ch ^ (row & 7)) << 4)]);
      }
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const int row = TN + wm * WM + f * 16 + lr;
        xf[f] = *reinterpret_cast<const uint4*>(&sc[buf][row * KSB + ((ch ^ (row & 7)) << 4)]);
      }
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) {
          if (j == 0) acc[a][b] = mma_fp4<0>(wf[a], xf[b], acc[a][b], sw[a], sx[b]);
          else acc[a][b] = mma_fp4<1>(wf[a], xf[b], acc[a][b], sw[a], sx[b]);
        }
    }

    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds Y[m][n .. n+3]
#pragma unroll
  for (int b = 0; b < FM; ++b) {
    const int m = m0 + wm * WM + b * 16 + lr;
    if (m >= g.m) continue;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
      const int n = n0 + wn * WN + a * 16 + 4 * lg;
      const v4f v = acc[a][b];
      if constexpr (BF16OUT) {
        uint16_t* yp = static_cast<uint16_t*>(g.y) + (int64_t)m * g.ld_y + n;
        if (y_vec && n + 3 < g.n) {
          const uint2 pk = make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                      bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
          *reinterpret_cast<uint2*>(yp) = pk;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < g.n) yp[r] = (uint16_t)bf16_bits(v[r]);
        }
      } else {
        float* yp = static_cast<float*>(g.y) + (int64_t)m * g.ld_y + n;
        if (y_vec && n + 3 < g.n) {
          *reinterpret_cast<float4*>(yp) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < g.n) yp[r] = v[r];
        }
      }
    }
  }
}

template <int TN, int TM, int WN, int WM>
hipError_t run(const GemmArgs& g, hipStream_t s) {
  constexpr int NT = (TN / WN) * (TM / WM) * 64;
  const int tiles = ((g.n + TN - 1) / TN) * ((g.m + TM - 1) / TM);
  const size_t ybytes = g.y_bf16 ? 2 : 4;
  const int y_vec = (((uintptr_t)g.y) % (4 * ybytes) == 0) && (g.ld_y % 4 == 0);
  const int s_vec = (((uintptr_t)g.a_scales) % 8 == 0) && (((uintptr_t)g.b_scales) % 8 == 0) &&
                    ((g.k / 32) % 8 == 0);
  if (g.y_bf16)
    gemm_kernel<TN, TM, WN, WM, true><<<tiles, NT, 0, s>>>(g, y_vec, s_vec);
  else
    gemm_kernel<TN, TM, WN, WM, false><<<tiles, NT, 0, s>>>(g, y_vec, s_vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.m == 0 || g.n == 0) return hipSuccess;
  if (gemm_small_supported(g)) return launch_gemm_small(g, s);
  if (g.tiled) return gemm_large_supported(g) ? launch_gemm_large(g, s) : hipErrorInvalidValue;
  if (g.m > 64 && gemm_large_supported(g)) return launch_gemm_large(g, s);
  return run<128, 128, 64, 64>(g, s);
}

}  // namespace mxfp4
