// Small-M MXFP4 x MXFP4 GEMM for gfx950 (decode shapes: M <= 64 activation
// rows against a large weight matrix).
//
// At decode sizes the layer is bound by reading the packed weights once from
// HBM: N*K/2 code bytes plus N*K/32 scale bytes, against 2*M*N*K FLOPs
// (arithmetic intensity ~ 3.8*M FLOP/B, far below the MFMA ridge).  The
// kernel reads the MXFP4 operands directly, with no dequantize pass ("AMD
// Quark delivers MXFP4 quantization for FLUX.1-dev on Instinct MI350 with
// 1.92x speedup", "MXFP4 quantization for diffusion models"; the decode
// setting is the LLM case of "Bridging the Gap Between Promise and
// Performance for Microscaling FP4 Quantization", "GPU Kernel Ondersteuning
// (QuTLASS)").
//
// MFMA: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1.  Lane l
// supplies row l % 16 of an operand and the 32-element block l / 16 of the
// instruction's 128-element K step as 16 packed bytes, plus that block's
// E8M0 byte (op_sel 0).  The result lane l holds D[4*(l/16) + r][l % 16].
//
// Design:
//  * One workgroup per 16 * NG weight rows (W is the MFMA's first operand, so
//    a lane ends with four consecutive output columns of one output row).  Its
//    waves split K into contiguous step ranges; a final LDS reduction sums the
//    waves' partial tiles.  NG = 2 (32 rows) while M <= 32: each activation
//    fragment then feeds two weight fragments, which halves the activation
//    reads from L2 -- at decode sizes those are as many bytes as the weights.
//  * Every operand fragment is exactly one MX block, loaded straight into
//    registers: 16 code bytes plus one scale byte per lane per K step.  A wave
//    issues all the loads of a chunk of 8 steps before its first MFMA, so the
//    whole weight matrix is in flight at once across the grid and the HBM
//    stream never waits on arithmetic.  Weights are read with non-temporal
//    loads (each byte is used once per call); the activation fragments are
//    shared by every workgroup and stay in L2.
//  * Row-major operands: a wave's code load covers 16 rows x 64 contiguous
//    bytes, and each lane loads its scale byte per step.  Tiled operands: one
//    K step of 16 rows is one contiguous 1 KiB run, and the scales of 4 steps
//    come in with one dword load per lane, spread to the lanes that use them
//    by a cross-lane permute (a quarter of the scale load instructions; the
//    scale loads were a third of the kernel's memory instructions).  Rows beyond M or N are clamped to a valid row (their results are
//    never stored); blocks beyond K are zero codes with a zero scale byte, so
//    a K tail contributes exactly 0.
//  * M is covered in groups of 16 rows that reuse the weight fragments held
//    in registers; past 64 rows, one grid row per 64 activation rows.  That
//    serves the small shapes too (fewer output tiles of 256 x 256 than the
//    chip has XCDs), where one large tile per workgroup would run a handful
//    of workgroups through a whole load ring and epilogue while the rest of
//    the chip idles.
//  * A wave whose chunk of steps lies wholly inside K issues its loads with
//    no predicates, so the waits before the MFMAs can count them down one by
//    one; only a K tail takes the predicated path.
#include "internal.h"
#include "block_quant.h"

#include <mutex>

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 8;      // K steps (128 elements each) per register chunk
constexpr int MAXW = 8;    // waves per workgroup (K split)
constexpr int MAXMG = 4;   // 16-row M groups (M <= 64)
constexpr int MAXACC = 4;  // NG * MG accumulator tiles per wave

__device__ __forceinline__ int tiled_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ v4f mma(const u32x4& a, const u32x4& b, const v4f& c, int sa, int sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 h = __builtin_convertvector(f2{a, b}, b2);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// Store Y[m][n .. n + 3] (bounds-checked against N) in the output dtype.
__device__ __forceinline__ void store4(const GemmArgs& g, int m, int n, const v4f& v, int y_vec) {
  if (g.y_bf16) {
    uint16_t* yp = static_cast<uint16_t*>(g.y) + (int64_t)m * g.ld_y + n;
    if (y_vec && n + 3 < g.n) {
      *reinterpret_cast<uint2*>(yp) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < g.n) yp[r] = (uint16_t)(pack_bf16(v[r], 0.f) & 0xFFFFu);
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

// Operand addressing for one lane: the fragment of K step s is 16 code bytes
// at code + s * cstride and one scale byte at scale + s * sstride.
struct Operand {
  const uint8_t* code;
  const uint8_t* scale;
  int64_t cstride, sstride;
  const uint8_t* scale_row;   // tiled: the row's 4 scale bytes of stage 0
};

template <bool TILED>
__device__ __forceinline__ Operand operand(const uint8_t* codes, const uint8_t* scales, int row,
                                           int rows, int k, int lg) {
  Operand o;
  if constexpr (TILED) {
    const int64_t nstage = k >> 7;
    const int64_t t = row >> 8;
    const int r = row & 255;
    o.code = codes + t * nstage * 16384 + r * 64 + 16 * (lg ^ tiled_swz(r));
    o.scale_row = scales + t * nstage * 1024 + r * 4;
    o.scale = o.scale_row + lg;
    o.cstride = 16384;
    o.sstride = 1024;
  } else {
    const int64_t rr = row < rows ? row : rows - 1;
    o.code = codes + rr * (k >> 1) + 16 * lg;
    o.scale = scales + rr * (k >> 5) + lg;
    o.scale_row = o.scale;
    o.cstride = 64;
    o.sstride = 4;
  }
  return o;
}

// Tiled operands: the scale bytes of one K step of a 16-row fragment are 64
// contiguous bytes (row-major [16][4]).  Lane (r, g) loads the dword of row r
// for step s0 + 4 i + g, i.e. the scales of all four blocks of that step; the
// scale of step s0 + 4 i + j for the lane's own block g then sits in byte g of
// lane (r, j)'s dword.  One dword load replaces four byte loads.
template <int NCH>
__device__ __forceinline__ void scales_dw(const Operand& o, int s0, int lane, int (&sc)[NCH]) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < NCH / 4; ++i) {
    const int dw = *reinterpret_cast<const int*>(o.scale_row + (int64_t)(s0 + 4 * i + lg) * o.sstride);
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[4 * i + j] = __shfl(dw, 16 * j + lr) >> (8 * lg);
  }
}

// MXFP4 output of the small-M kernel: Y requantized per 32-block along N by
// the quantizer's rule, from the same fp32 sums that the fp32 output stores.
// The workgroup's 32 weight rows (NG = 2) are one block of each output row:
// lane (r, g) holds columns 4g .. 4g + 3 of fragment 0 (v0) and of fragment 1
// (v1), i.e. code bytes 2g, 2g + 1 and 8 + 2g, 8 + 2g + 1 of row r's block.
// The block amax comes from the four lanes of row r (an exact max), the codes
// from the E2M1 converter at the block scale, and lane (r, 0) gathers the 16
// code bytes and stores them with the scale byte.
__device__ __forceinline__ void store_requant(const GemmArgs& g, int m, int n0, const v4f& v0, const v4f& v1,
                                              int lane) {
  float am = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) am = fmaxf(am, fmaxf(fabsf(v0[r]), fabsf(v1[r])));
  am = fmaxf(am, __shfl_xor(am, 16));
  am = fmaxf(am, __shfl_xor(am, 32));
  const uint32_t sbyte = blockq::sbyte_of_amax(am);
  const float sc = blockq::scale_of(sbyte);
  uint32_t w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v0[0], v0[1], sc, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v0[2], v0[3], sc, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v1[0], v1[1], sc, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v1[2], v1[3], sc, 1);
  const int lr = lane & 15;
  uint32_t p0[4], p1[4];   // the low 16 bits of w0, w1 of lanes (r, 0..3)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p0[j] = (uint32_t)__shfl((int)w0, lr + 16 * j) & 0xFFFFu;
    p1[j] = (uint32_t)__shfl((int)w1, lr + 16 * j) & 0xFFFFu;
  }
  if ((lane >> 4) != 0 || m >= g.m) return;
  const uint4 codes = make_uint4(p0[0] | (p0[1] << 16), p0[2] | (p0[3] << 16), p1[0] | (p1[1] << 16),
                                 p1[2] | (p1[3] << 16));
  const int blk = n0 >> 5;
  if (g.q_tiled) {
    const uint32_t r8 = (uint32_t)m & 255u, c = (uint32_t)blk & 3u;
    const uint64_t ts = (uint64_t)((uint32_t)m >> 8) * ((uint32_t)g.n >> 7) + ((uint32_t)blk >> 2);
    *reinterpret_cast<uint4*>(g.q_codes + ts * 16384 + r8 * 64 + 16 * (c ^ tiled_swz((int)r8))) = codes;
    g.q_scales[ts * 1024 + r8 * 4 + c] = (uint8_t)sbyte;
  } else {
    *reinterpret_cast<uint4*>(g.q_codes + (int64_t)m * (g.n >> 1) + 16 * blk) = codes;
    g.q_scales[(int64_t)m * (g.n >> 5) + blk] = (uint8_t)sbyte;
  }
}

// OUT: 0 fp32 Y, 1 bf16 Y, 2 MXFP4 Y (NG == 2: one 32-block of each output
// row per workgroup).
template <int MG, int NG, int OUT, bool TILED>
__global__ __launch_bounds__(64 * MAXW) void gemm_small_kernel(GemmArgs g, int spw, int y_vec) {
  static_assert(MG * NG <= 2 * MAXACC, "reduction buffer size");
  static_assert(OUT != 2 || NG == 2, "the MXFP4 output needs 32 weight rows per workgroup");
  static_assert(CH % 4 == 0, "dword scale loads cover 4 steps");
  constexpr bool BF16OUT = OUT == 1;
  __shared__ v4f red[MAXW][MG * NG][64];

  const int lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16 * NG;
  const int m0 = blockIdx.y * 16 * MAXMG;   // M beyond 64 rows: one grid row per 64 activation rows
  const int kblocks = g.k >> 5;
  const int nsteps = (g.k + 127) >> 7;
  const int s_begin = wave * spw;
  const int s_end = min(nsteps, s_begin + spw);

  Operand w[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) w[q] = operand<TILED>(g.b_codes, g.b_scales, n0 + 16 * q + lr, g.n, g.k, lg);
  Operand x[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) x[mg] = operand<TILED>(g.a_codes, g.a_scales, m0 + 16 * mg + lr, g.m, g.k, lg);

  v4f acc[NG][MG];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) acc[q][mg] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int s0 = s_begin; s0 < s_end; s0 += CH) {
    // every step of the chunk inside this wave's range and inside K
    const bool full = s0 + CH <= s_end && (TILED || 4 * (s0 + CH) <= kblocks);
    u32x4 wf[NG][CH];
    int ws[NG][CH];
    if (full) {
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          wf[q][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w[q].code + (s0 + j) * w[q].cstride));
          if constexpr (!TILED) ws[q][j] = w[q].scale[(s0 + j) * w[q].sstride];
        }
      if constexpr (TILED) {
#pragma unroll
        for (int q = 0; q < NG; ++q) scales_dw<CH>(w[q], s0, lane, ws[q]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const int s = s0 + j;
          wf[q][j] = u32x4{0u, 0u, 0u, 0u};
          ws[q][j] = 0;
          if (s < s_end && (TILED || 4 * s + lg < kblocks)) {
            wf[q][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w[q].code + s * w[q].cstride));
            ws[q][j] = w[q].scale[s * w[q].sstride];
          }
        }
    }
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      u32x4 xf[CH];
      int xs[CH];
      if (full) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          xf[j] = *reinterpret_cast<const u32x4*>(x[mg].code + (s0 + j) * x[mg].cstride);
          if constexpr (!TILED) xs[j] = x[mg].scale[(s0 + j) * x[mg].sstride];
        }
        if constexpr (TILED) scales_dw<CH>(x[mg], s0, lane, xs);
      } else {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const int s = s0 + j;
          xf[j] = u32x4{0u, 0u, 0u, 0u};
          xs[j] = 0;
          if (s < s_end && (TILED || 4 * s + lg < kblocks)) {
            xf[j] = *reinterpret_cast<const u32x4*>(x[mg].code + s * x[mg].cstride);
            xs[j] = x[mg].scale[s * x[mg].sstride];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < CH; ++j)
        if (s0 + j < s_end) {
#pragma unroll
          for (int q = 0; q < NG; ++q) acc[q][mg] = mma(wf[q][j], xf[j], acc[q][mg], ws[q][j], xs[j]);
        }
    }
  }

  // lane holds Y[m0 + 16 mg + lr][n .. n + 3] of weight group q
  auto store_frag = [&](int q, int mg, const v4f& v) {
    const int n = n0 + 16 * q + 4 * lg;
    const int m = m0 + 16 * mg + lr;
    if (m >= g.m) return;
    if constexpr (BF16OUT) {
      uint16_t* yp = static_cast<uint16_t*>(g.y) + (int64_t)m * g.ld_y + n;
      if (y_vec && n + 3 < g.n) {
        *reinterpret_cast<uint2*>(yp) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < g.n) yp[r] = (uint16_t)(pack_bf16(v[r], 0.f) & 0xFFFFu);
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
  };

  // The waves' partial tiles are summed in wave order (wave 0's, then wave
  // 1's, ...).  MXFP4 output: wave 0 sums and requantizes the 32-row block.
  // Otherwise each fragment is summed and stored by one wave, so the sums and
  // stores of the tile's fragments run on several waves at once.
  if (nwaves > 1) {
    if constexpr (OUT == 2) {
      if (wave > 0) {
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
          for (int mg = 0; mg < MG; ++mg) red[wave][q * MG + mg][lane] = acc[q][mg];
      }
      __syncthreads();
      if (wave > 0) return;
      for (int w2 = 1; w2 < nwaves; ++w2) {
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
          for (int mg = 0; mg < MG; ++mg) acc[q][mg] += red[w2][q * MG + mg][lane];
      }
    } else {
#pragma unroll
      for (int q = 0; q < NG; ++q)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) red[wave][q * MG + mg][lane] = acc[q][mg];
      __syncthreads();
      for (int f = wave; f < MG * NG; f += nwaves) {
        v4f sum = red[0][f][lane];
        for (int w2 = 1; w2 < nwaves; ++w2) sum += red[w2][f][lane];
        store_frag(f / MG, f % MG, sum);
      }
      return;
    }
  }

  if constexpr (OUT == 2) {
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) store_requant(g, m0 + 16 * mg + lr, n0, acc[0][mg], acc[NG - 1][mg], lane);
    return;
  } else {
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) store_frag(q, mg, acc[q][mg]);
  }
}

template <int MG, int NG, int OUT, bool TILED>
void launch(const GemmArgs& g, int nwaves, int spw, int y_vec, hipStream_t s) {
  const dim3 grid((g.n + 16 * NG - 1) / (16 * NG), (g.m + 16 * MAXMG - 1) / (16 * MAXMG));
  gemm_small_kernel<MG, NG, OUT, TILED><<<grid, 64 * nwaves, 0, s>>>(g, spw, y_vec);
}

template <int MG, int NG>
void launch_mg(const GemmArgs& g, int nwaves, int spw, int y_vec, hipStream_t s) {
  if (g.q_out) {
    if (g.tiled) launch<MG, 2, 2, true>(g, nwaves, spw, y_vec, s);
    else launch<MG, 2, 2, false>(g, nwaves, spw, y_vec, s);
  } else if (g.y_bf16) {
    if (g.tiled) launch<MG, NG, 1, true>(g, nwaves, spw, y_vec, s);
    else launch<MG, NG, 1, false>(g, nwaves, spw, y_vec, s);
  } else {
    if (g.tiled) launch<MG, NG, 0, true>(g, nwaves, spw, y_vec, s);
    else launch<MG, NG, 0, false>(g, nwaves, spw, y_vec, s);
  }
}


// ---------------------------------------------------------------------------
// Fused small-M linear layer: Y = Q(rot(X)) * W^T in one launch, with the
// activation rotation and quantization done inside the GEMM kernel (the
// rotation fused into the quantization and the matmul, as in "Bridging the
// Gap Between Promise and Performance for Microscaling FP4 Quantization",
// "GPU Kernel Ondersteuning (QuTLASS)").
//
// The compute waves are those of gemm_small_kernel: K split over the waves
// in chunks of CH steps (the same split), the same MFMA chains and the same
// LDS reduction, so Y equals mxfp4_quantize_rotate followed by mxfp4_gemm
// bit for bit.  A compute workgroup takes 16 NG weight rows and has one more
// wave, its sync wave.
//  * Producers rotate and quantize X.  A pass takes one unit of 16 rows x 128
//    elements (one K step of one M group), one block per lane, with the
//    quantizer's own arithmetic (block_quant.h).  The codes and scales go
//    into the workspace already in MFMA operand order, through
//    device-coherent (sc1) stores that write through the XCD's L2.  A
//    producer wave waits for its stores, then counts itself on a
//    device-scope counter, kept in 16 copies on separate lines.
//  * Where the compute grid leaves CUs idle and they have a wave for every
//    unit (the decode shapes: 224 workgroups on 256 CUs), the producers are
//    `pwg` extra workgroups ahead of the compute ones, one per idle CU.  A
//    CU's vector memory requests are served in order, so a producer sharing
//    its CU with four compute waves waited behind their weight loads: its
//    block, its store acknowledgements and its count each took microseconds
//    longer.  On a CU of their own the layer took 9.1 instead of 10.4 us at
//    16 x 4096 -> 14336.  Otherwise the sync waves of the first `nprod`
//    compute workgroups produce, and the compute waves hold back their
//    weight stream for about 0.4 us so that the producers' loads go first.
//  * Every sync wave polls one copy of that counter until all producers have
//    counted, then releases its workgroup's compute waves at a barrier.
//    (With one copy, the increments queued behind a couple of hundred
//    pollers of the same address: 2.4 us from the last increment to the
//    polls seeing it.)
//  * The compute waves issue their first chunk of weight loads before that
//    barrier, so the weight stream (the layer's HBM-bound part) runs while X
//    is quantized and handed over.  After the barrier they read the
//    quantized X with device-scope coherent loads (the coherence the compiler
//    gives agent-scope atomic loads, so no copy of a line from an earlier
//    call is returned; the fetch counters show these reads served inside the
//    XCDs' L2) and run the MFMAs as the weights arrive.
// The compute waves never poll themselves.  A wave's vector loads complete
// in order, so a poll issued behind a weight chunk would wait for all of it.
// A workgroup that waits holds its CU, and a workgroup of 5 or 9 waves takes
// a CU's wave slots (one per SIMD per 4 waves, rounded up, at the register
// budget of these kernels).  So up to 4 compute waves and 16 activation rows
// take 64 weight rows per workgroup (224 workgroups for 14336 rows, all
// resident at once); a grid larger than the CU count still completes, the
// later workgroups starting as the first ones finish, but takes about a
// second round.
//
// Termination.  Producers wait on nothing before they count, and they are
// in the lowest-numbered workgroups, which the dispatcher places first.  The
// poll is bounded all the same (2^20 polls, tens of milliseconds); past the
// bound the sync wave sets an error word in the workspace and goes on, and
// that call's Y is undefined.
//
// Reset.  Once its compute waves are released, each sync wave counts itself
// on the counter of its group of workgroups; the last of a group clears that
// counter and counts the group on a top counter, and the last group clears
// the top counter and the producer counts.  So every counter is zero
// whenever the kernel has completed, and calls in stream order can share one
// workspace.  (One counter for the whole grid serialized several hundred
// atomics on one address: about 2 us.)
constexpr int LPROD_MAX = 256;               // producer workgroups at most (one unit each up to there)
constexpr uint32_t LPOLL_LIMIT = 1u << 20;   // polls before a sync wave gives up
constexpr int LLINE = 32;                    // counter words 128 bytes apart
constexpr int LREPL = 16;                    // copies of the producer count, one line each
constexpr int CNT_PRODUCED = 0, CNT_ERROR = LREPL * LLINE, CNT_TOP = CNT_ERROR + LLINE, CNT_GROUP0 = CNT_TOP + LLINE;
constexpr int LGROUPS_MAX = (int)(kLinearCounterBytes / 4 / LLINE) - LREPL - 2;
constexpr int kCoherent = 16;                // buffer cache policy sc1: device scope

template <bool XBF16>
struct RawBlock {
  u32x4 c[XBF16 ? 4 : 8];
};

template <bool XBF16>
__device__ __forceinline__ void load_block(const uint8_t* p, bool ok, RawBlock<XBF16>& b) {
#pragma unroll
  for (int i = 0; i < (XBF16 ? 4 : 8); ++i)
    b.c[i] = ok ? *reinterpret_cast<const u32x4*>(p + 16 * i) : u32x4{0u, 0u, 0u, 0u};
}

template <bool XBF16, int ROT, int P, int Q>
__device__ __forceinline__ void quantize_raw(const RawBlock<XBF16>& b, const float* fa, const float* fb, u32x4& codes,
                                             int& sbyte) {
  float v[32];
  if constexpr (XBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = blockq::bf16_lo(b.c[i][j]);
        v[8 * i + 2 * j + 1] = blockq::bf16_hi(b.c[i][j]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = __uint_as_float(b.c[i][j]);
  }
  blockq::rotate_block<ROT, P, Q>(fa, fb, v);
  uint32_t w[4];
  sbyte = (int)blockq::encode_block(v, w);
  codes = u32x4{w[0], w[1], w[2], w[3]};
}

// Workspace image of the quantized activations: unit u = mg * nsteps + s
// (M group mg, K step s) holds 64 lanes x 16 code bytes at 1024 u -- lane l
// the block l / 16 of row l % 16, as the MFMA reads it -- and, at
// 1024 units + 128 u, the scale bytes as 16 dwords, dword r holding the
// step's four block scales of row r (the layout scales_dw reads).
__device__ __forceinline__ uint32_t xq_code_off(int u, int lane) { return ((uint32_t)u * 64u + lane) * 16u; }
__device__ __forceinline__ uint32_t xq_scale_off(int units, int u, int row) {
  return (uint32_t)units * 1024u + (uint32_t)u * 128u + 4u * row;
}

// A producer wave: quantize units first, first + stride, ... of X into the
// workspace, then count itself once its stores have completed.
template <int ROT, int P, int Q>
__device__ __forceinline__ void produce(const LinearArgs& L, const __amdgpu_buffer_rsrc_t& xr, int units, int nsteps,
                                        int kblocks, int first, int stride, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const uint8_t* xb = static_cast<const uint8_t*>(L.x);
  // Kronecker factors (4 x 8 and 8 x 4: 80 values) are read before the first
  // block and ahead of the compute waves' weight stream.  Read where the
  // chains first use them, these uniform loads were issued after the block
  // had arrived and then waited microseconds behind the weight loads.
  constexpr bool FPRE = ROT == 2 && P * P + Q * Q <= 80;
  float fa_r[FPRE ? P * P : 1], fb_r[FPRE ? Q * Q : 1];
  if constexpr (FPRE) {
#pragma unroll
    for (int i = 0; i < P * P; ++i) fa_r[i] = L.fa[i];
#pragma unroll
    for (int i = 0; i < Q * Q; ++i) fb_r[i] = L.fb[i];
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int u = first; u < units; u += stride) {
    const int mg = u / nsteps, s = u - mg * nsteps;
    const int row = 16 * mg + lr, c = 4 * s + lg;
    const bool ok = row < L.g.m && c < kblocks;
    RawBlock<true> raw;
    load_block<true>(xb + ((int64_t)(ok ? row : 0) * L.ld_x + (int64_t)(ok ? c : 0) * 32) * 2, ok, raw);
    u32x4 codes;
    int sb;
    quantize_raw<true, ROT, P, Q>(raw, ROT == 3 ? L.fa + 32 * min(c, kblocks - 1) : (FPRE ? fa_r : L.fa),
                                  FPRE ? fb_r : L.fb, codes, sb);
    if (!ok) {   // rows past M and blocks past K: zero codes, zero scale byte
      codes = u32x4{0u, 0u, 0u, 0u};
      sb = 0;
    }
    __builtin_amdgcn_raw_buffer_store_b128(codes, xr, (int)xq_code_off(u, lane), 0, kCoherent);
    int d = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) d |= (__shfl(sb, lr + 16 * j) & 0xFF) << (8 * j);
    if (lg == 0) __builtin_amdgcn_raw_buffer_store_b32(d, xr, (int)xq_scale_off(units, u, lr), 0, kCoherent);
  }
  // the stores have reached the device-coherent level before the count,
  // which goes to every copy (lane i counts copy i)
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
  if (lane < LREPL)
    __hip_atomic_fetch_add(L.counters + CNT_PRODUCED + LLINE * lane, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// WB: waves per workgroup the kernel is compiled for (compute waves + 1).
template <int MG, int NG, int WB, int ROT, int P, int Q, bool TILED>
__global__ __launch_bounds__(64 * WB) void linear_small_kernel(LinearArgs L, int nwaves, int spw, int nprod,
                                                                 int ncount, int pwg, int gsize, int y_vec) {
  static_assert(MG * NG <= 2 * MAXACC, "reduction buffer size");
  static_assert(CH % 4 == 0, "dword scale loads cover 4 steps");
  __shared__ v4f red[MAXW][MG * NG][64];
  __shared__ uint32_t red_ready;   // compute waves whose partial tile is in red
  // Tiled weights, one M group, 64 rows per workgroup (at most 4 compute
  // waves, so at most 32 K steps): the sync wave loads the workgroup's weight
  // scales into LDS at the start, 8 one-KiB loads, instead of 32 dword loads
  // by the compute waves behind their weight codes (9.09 -> 8.99 us at
  // 16 x 4096 -> 14336 with Kron 4 x 8, bit-identical).
  constexpr bool SL = TILED && MG == 1 && NG == 4;
  __shared__ __attribute__((aligned(16))) uint32_t wsl[SL ? 32 : 1][64];
  const GemmArgs& g = L.g;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int cb = (int)blockIdx.x - pwg;   // compute workgroup index
  const int kblocks = g.k >> 5;
  const int nsteps = (g.k + 127) >> 7;
  const int units = MG * nsteps;
  const bool compute = wave < nwaves;
  if (threadIdx.x == 0) {
    red_ready = 0u;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): in LDS before the barrier below
  }
  const int s_begin = wave * spw;
  const int s_end = min(nsteps, s_begin + spw);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(L.xq, 0, units * 1152, 0x00020000);
  if (cb < 0) {
    // producer workgroup, on a CU with no weight stream: each wave with
    // units quantizes them and counts itself
    const int first = wave * pwg + (int)blockIdx.x;
    if (first < units) produce<ROT, P, Q>(L, xr, units, nsteps, kblocks, first, pwg * (nwaves + 1), lane);
    return;
  }
  const int n0 = cb * 16 * NG;

  Operand w[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) w[q] = operand<TILED>(g.b_codes, g.b_scales, n0 + 16 * q + lr, g.n, g.k, lg);
  v4f acc[NG][MG];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) acc[q][mg] = v4f{0.f, 0.f, 0.f, 0.f};

  // One chunk of this wave's weights, as gemm_small_kernel loads it.  Tiled
  // scales stay packed (wsd: the dwords scales_dw loads), each spread to its
  // lanes right before its MFMA, which keeps 24 registers free for the
  // weight codes in flight.
  u32x4 wf[NG][CH];
  int ws[NG][CH];
  int wsd[NG][CH / 4];
  auto load_weights = [&](int s0) {
    if constexpr (TILED && !SL) {   // steps past the range (never used) read the last step's dword
#pragma unroll
      for (int q = 0; q < NG; ++q)
#pragma unroll
        for (int i = 0; i < CH / 4; ++i)
          wsd[q][i] = *reinterpret_cast<const int*>(w[q].scale_row +
                                                    (int64_t)min(s0 + 4 * i + lg, nsteps - 1) * w[q].sstride);
    }
    const bool full = s0 + CH <= s_end && (TILED || 4 * (s0 + CH) <= kblocks);
    if (full) {
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          wf[q][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w[q].code + (s0 + j) * w[q].cstride));
          if constexpr (!TILED) ws[q][j] = w[q].scale[(s0 + j) * w[q].sstride];
        }
    } else {
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const int s = s0 + j;
          wf[q][j] = u32x4{0u, 0u, 0u, 0u};
          ws[q][j] = 0;
          if (s < s_end && (TILED || 4 * s + lg < kblocks)) {
            wf[q][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w[q].code + s * w[q].cstride));
            if constexpr (!TILED) ws[q][j] = w[q].scale[s * w[q].sstride];
          }
        }
    }
  };
  int s0c = 0;   // first step of the chunk being computed
  // the scale byte of weight fragment q at step s0 + j (in the low 8 bits)
  auto wscale = [&](int q, int j) -> int {
    if constexpr (SL)
      return (int)reinterpret_cast<const uint8_t*>(&wsl[0][0])[(s0c + j) * 256 + (16 * q + lr) * 4 + lg];
    else if constexpr (TILED) return __shfl(wsd[q][j >> 2], 16 * (j & 3) + lr) >> (8 * lg);
    else return ws[q][j];
  };

  // The compute waves and the sync wave meet at one barrier, each on its own
  // path (no register of one path is live on the other).  A bare barrier: a
  // workgroup fence would wait for the weight loads in flight.
  if (compute) {
    // With producers in the compute workgroups, the weight stream starts
    // about 0.4 us after their first loads.  Issued at once, it filled the
    // memory queues ahead of those loads, and the producers' blocks, factors
    // and store acknowledgements waited behind it (a producer's block arrived
    // after 4.8 us instead of 1.9).  Producers on CUs of their own need no
    // delay (with it: 9.5 instead of 9.1 us).
    if (pwg == 0) __builtin_amdgcn_s_sleep(16);
    if (s_begin < s_end) load_weights(s_begin);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");   // keeps the activation loads below the barrier
    __builtin_amdgcn_sched_barrier(0);
    for (int s0 = s_begin; s0 < s_end; s0 += CH) {
      if (s0 != s_begin) load_weights(s0);
      s0c = s0;
      // One M group: the weight scales spread now, before the activation
      // loads (from LDS with tiled weights; dword loads, which wait for the
      // chunk, with row-major ones: 11.2 instead of 11.6 us at 16 x 4096 ->
      // 14336 when those were the tiled path too).  More M groups: spread at
      // each MFMA, so that the first group's activation loads go out before
      // the weights are in (18.8 instead of 21.8 us at 64 rows).
      int wsv[NG][CH];
      if constexpr (MG == 1) {
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
          for (int j = 0; j < CH; ++j) wsv[q][j] = wscale(q, j);
      }
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        u32x4 xf[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const int st = min(s0 + j, nsteps - 1);   // steps past the range are not used
          xf[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xq_code_off(mg * nsteps + st, lane), 0, kCoherent);
        }
        int xsd[CH / 4];
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) {
          const int st = min(s0 + 4 * i + lg, nsteps - 1);
          xsd[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(xr, (int)xq_scale_off(units, mg * nsteps + st, lr), 0,
                                                             kCoherent);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j)
          if (s0 + j < s_end) {
            const int xs = __shfl(xsd[j >> 2], 16 * (j & 3) + lr) >> (8 * lg);
#pragma unroll
            for (int q = 0; q < NG; ++q)
              acc[q][mg] = mma(wf[q][j], xf[j], acc[q][mg], MG == 1 ? wsv[q][j] : wscale(q, j), xs);
          }
      }
    }
  } else {
    if constexpr (SL) {
      // the workgroup's 64 rows of one tiled stage are 256 contiguous scale
      // bytes; one 1 KiB load takes 4 steps (steps past the end re-read the
      // last one into rows of wsl that are never used)
      const uint8_t* sb = g.b_scales + (int64_t)(n0 >> 8) * nsteps * 1024 + (n0 & 255) * 4 + 16 * (lane & 15);
      for (int i = 0; 4 * i < nsteps; ++i)
        __builtin_amdgcn_global_load_lds(sb + (int64_t)min(4 * i + (lane >> 4), nsteps - 1) * 1024,
                                         reinterpret_cast<uint8_t*>(&wsl[4 * i][0]), 16, 0, 0);
    }
    if (cb < nprod) produce<ROT, P, Q>(L, xr, units, nsteps, kblocks, cb, nprod, lane);
    if (lane == 0) {
      const uint32_t* cnt = L.counters + CNT_PRODUCED + LLINE * (cb % LREPL);
      uint32_t polls = 0;
      while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)ncount) {
        __builtin_amdgcn_s_sleep(1);
        if (++polls == LPOLL_LIMIT) {
          __hip_atomic_store(L.counters + CNT_ERROR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    if constexpr (SL) __builtin_amdgcn_s_waitcnt(0);   // the scales are in LDS
    __builtin_amdgcn_s_barrier();   // releases the compute waves
    if (lane == 0) {
      // this workgroup is past its poll: count it; the last one clears
      const int ncomp = (int)gridDim.x - pwg;
      const int grp = cb / gsize;
      const uint32_t members = (uint32_t)min(gsize, ncomp - grp * gsize);
      const uint32_t ngroups = (ncomp + gsize - 1) / gsize;
      uint32_t* gc = L.counters + CNT_GROUP0 + LLINE * grp;
      if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
        __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__hip_atomic_fetch_add(L.counters + CNT_TOP, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            ngroups - 1) {
          __hip_atomic_store(L.counters + CNT_TOP, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int r = 0; r < LREPL; ++r)
            __hip_atomic_store(L.counters + CNT_PRODUCED + LLINE * r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // The compute waves' partial tiles summed in wave order (wave 0's, then
  // wave 1's, ...), as gemm_small_kernel does, but each fragment summed and
  // stored by one wave: every compute wave parks its partial tile in LDS and
  // counts itself, waits for the count of all compute waves (an LDS count, not
  // a workgroup barrier, which would also wait for the sync wave's counter
  // round trips), then sums and stores fragments wave, wave + nwaves, ...
  if (!compute) return;
  if (nwaves == 1) {
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        const int m = 16 * mg + lr;
        if (m < g.m) store4(g, m, n0 + 16 * q + 4 * lg, acc[q][mg], y_vec);
      }
    return;
  }
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) red[wave][q * MG + mg][lane] = acc[q][mg];
  if (lane == 0) __hip_atomic_fetch_add(&red_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  // bounded: the compute waves wait on nothing once their loads are in (the
  // bound is far beyond any real wait)
  for (uint32_t spins = 0;
       __hip_atomic_load(&red_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)nwaves &&
       spins < (1u << 24);
       ++spins)
    __builtin_amdgcn_s_sleep(1);
  for (int f = wave; f < MG * NG; f += nwaves) {
    v4f sum = red[0][f][lane];
    for (int w2 = 1; w2 < nwaves; ++w2) sum += red[w2][f][lane];
    const int m = 16 * (f % MG) + lr;
    if (m < g.m) store4(g, m, n0 + 16 * (f / MG) + 4 * lg, sum, y_vec);
  }
}

// K split over the waves: chunks of CH steps, up to MAXW waves (the fused
// layer takes the same split as the small-M GEMM, so their sums agree)
void wave_split(int k, int& nwaves, int& spw) {
  const int nsteps = (k + 127) / 128;
  nwaves = (nsteps + CH - 1) / CH;
  if (nwaves > MAXW) nwaves = MAXW;
  if (nwaves < 1) nwaves = 1;
  spw = (nsteps + nwaves - 1) / nwaves;
}

template <int MG, int NG, int WB, int ROT, int P, int Q>
void launch_fused(const LinearArgs& L, int nwaves, int spw, int y_vec, hipStream_t s) {
  const int grid = (L.g.n + 16 * NG - 1) / (16 * NG);
  const int units = MG * ((L.g.k + 127) / 128);
  // producer workgroups on the CUs the compute grid leaves idle, if they
  // have a wave for every unit; else producers in the compute workgroups
  const int idle = cu_count() - grid;
  const int pwg = idle > 0 && idle * (nwaves + 1) >= units ? min(idle, units) : 0;
  const int nprod = pwg ? 0 : min(min(units, grid), LPROD_MAX);
  const int ncount = pwg ? min(units, pwg * (nwaves + 1)) : nprod;
  const int gsize = max(32, (grid + LGROUPS_MAX - 1) / LGROUPS_MAX);
  const int threads = 64 * (nwaves + 1);
  if (L.g.tiled)
    linear_small_kernel<MG, NG, WB, ROT, P, Q, true><<<grid + pwg, threads, 0, s>>>(L, nwaves, spw, nprod, ncount, pwg,
                                                                                    gsize, y_vec);
  else
    linear_small_kernel<MG, NG, WB, ROT, P, Q, false><<<grid + pwg, threads, 0, s>>>(L, nwaves, spw, nprod, ncount, pwg,
                                                                                     gsize, y_vec);
}

// Up to 4 compute waves (k <= 4096): a register budget of two waves per
// SIMD, which holds a chunk of 64 weight rows for one M group (32 rows for
// more); past 4 compute waves, three waves per SIMD and half the rows.
template <int MG, int ROT, int P, int Q>
void launch_fused_waves(const LinearArgs& L, int y_vec, hipStream_t s) {
  int nwaves, spw;
  wave_split(L.g.k, nwaves, spw);
  if (nwaves <= 4) launch_fused<MG, MG == 1 ? 4 : 2, 5, ROT, P, Q>(L, nwaves, spw, y_vec, s);
  else launch_fused<MG, MG <= 2 ? 2 : 1, MAXW + 1, ROT, P, Q>(L, nwaves, spw, y_vec, s);
}

template <int MG>
hipError_t launch_fused_mg(const LinearArgs& L, int y_vec, hipStream_t s) {
  if (L.rot == 0) launch_fused_waves<MG, 0, 1, 32>(L, y_vec, s);
  else if (L.rot == 1) launch_fused_waves<MG, 1, 1, 32>(L, y_vec, s);
  else if (L.rot == 3) launch_fused_waves<MG, 3, 1, 32>(L, y_vec, s);
  else {
    switch (L.p) {
      case 2: launch_fused_waves<MG, 2, 2, 16>(L, y_vec, s); break;
      case 4: launch_fused_waves<MG, 2, 4, 8>(L, y_vec, s); break;
      case 8: launch_fused_waves<MG, 2, 8, 4>(L, y_vec, s); break;
      case 16: launch_fused_waves<MG, 2, 16, 2>(L, y_vec, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipSuccess;
}

}  // namespace

// The small-M kernel takes decode shapes (m <= 64) and shapes with fewer
// 256 x 256 output tiles than the chip has XCDs (8), where the large-tile
// kernel would run a handful of workgroups through its whole load ring and
// epilogue while the rest of the chip idles; here each workgroup takes 32
// (16) weight rows and 64 activation rows.
bool gemm_small_route(int64_t m, int64_t n) {
  return m >= 1 && (m <= 16 * MAXMG || ((m + 255) / 256) * ((n + 255) / 256) < 8);
}

bool gemm_small_supported(const GemmArgs& g) {
  return gemm_small_route(g.m, g.n) && (!g.q_out || (g.n % (g.q_tiled ? 128 : 32)) == 0);
}

bool linear_small_supported(const LinearArgs& L) {
  return L.g.m >= 1 && L.g.m <= 16 * MAXMG && L.x_bf16 && (L.rot != 2 || (L.p >= 2 && L.p <= 16));
}

hipError_t launch_gemm_small(const GemmArgs& g, hipStream_t s) {
  if (!gemm_small_supported(g)) return hipErrorInvalidValue;
  int nwaves, spw;
  wave_split(g.k, nwaves, spw);
  const size_t ybytes = g.y_bf16 ? 2 : 4;
  const int y_vec = (((uintptr_t)g.y) % (4 * ybytes) == 0) && (g.ld_y % 4 == 0);
  switch (g.m > 16 * MAXMG ? MAXMG : (g.m + 15) / 16) {
    case 1: launch_mg<1, 2>(g, nwaves, spw, y_vec, s); break;
    case 2: launch_mg<2, 2>(g, nwaves, spw, y_vec, s); break;
    case 3: launch_mg<3, 1>(g, nwaves, spw, y_vec, s); break;
    default: launch_mg<4, 1>(g, nwaves, spw, y_vec, s); break;
  }
  return hipGetLastError();
}

}  // namespace mxfp4

namespace mxfp4 {

// ---------------------------------------------------------------------------
// Fixed device scratch for mxfp4_linear_small_noalloc, the fused layer for
// callers that cannot allocate: the fused layer's workspace lives in this
// array, one copy per GPU, held until the process ends.  Host code never
// uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[kLinearStaticScratchBytes];

__global__ void clear_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t linear_small_static_scratch(void** ptr, hipStream_t s) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // the counters start at zero (a fill kernel, not a memset node, in case
    // the first call is captured into a graph); later calls leave them zero
    constexpr int words = (int)(kLinearCounterBytes / 4);
    clear_words_kernel<<<(words + 255) / 256, 256, 0, s>>>(static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int64_t linear_small_workspace_bytes(int64_t m, int64_t k) {
  const int64_t units = (m + 15) / 16 * ((k + 127) / 128);
  return kLinearCounterBytes + units * 1152;
}

hipError_t launch_linear_small(const LinearArgs& L, hipStream_t s) {
  if (!linear_small_supported(L) || L.counters == nullptr || L.xq == nullptr) return hipErrorInvalidValue;
  const size_t ybytes = L.g.y_bf16 ? 2 : 4;
  const int y_vec = (((uintptr_t)L.g.y) % (4 * ybytes) == 0) && (L.g.ld_y % 4 == 0);
  hipError_t e;
  switch ((L.g.m + 15) / 16) {
    case 1: e = launch_fused_mg<1>(L, y_vec, s); break;
    case 2: e = launch_fused_mg<2>(L, y_vec, s); break;
    case 3: e = launch_fused_mg<3>(L, y_vec, s); break;
    default: e = launch_fused_mg<4>(L, y_vec, s); break;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace mxfp4
