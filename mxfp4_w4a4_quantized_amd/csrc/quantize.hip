// Online MXFP4 activation quantizer for gfx950 (CDNA4).
//
// Each lane owns one 32-element block.  A wave first loads its 64 blocks with
// contiguous 1 KiB loads (lane l reads 16-byte chunk l of each KiB, so every
// load instruction is fully coalesced), parks them in a wave-private LDS
// slab, and then each lane reads back its own block.  In the slab, chunk q of
// block i sits at chunk position q ^ f(i) of the block's row, so both the
// coalesced writes and the per-block reads hit distinct banks.  The lane then
// widens to fp32, applies the optional block rotation entirely in registers,
// reduces the block amax, derives the E8M0 scale from the amax exponent bits,
// converts pairs of values with the hardware E2M1 converter, whose scale
// operand is the block scale (v_cvt_scalef32_pk_fp4_f32: divide by the
// power-of-two scale, round to nearest even, saturate, keep the sign on zero) and writes its 16 code bytes with one 16-byte store (consecutive
// lanes, consecutive blocks) and its scale with one byte store.  X is read
// once, with non-temporal loads.
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
//
// Small inputs with a Kronecker transform (at most 16384 blocks, p <= 16) use a
// second kernel that spreads each block's transform over q lanes (below).
#include "internal.h"
#include "block_quant.h"

namespace mxfp4 {
namespace {

using namespace blockq;

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Chunk swizzle inside the LDS slab: a block is CPB 16-byte chunks; the
// 16 lanes of one ds_read_b128 phase read chunk q of 16 consecutive blocks,
// which land in 16 distinct 16-byte bank groups of the 64-bank LDS.
template <int CPB>
__device__ __forceinline__ int slab_swz(int blk) {
  return CPB == 4 ? (blk >> 2) & 3 : (blk >> 1) & 7;
}

// Tiled-layout chunk swizzle (the GEMM's LDS bank swizzle, baked into the
// tiled codes): block c of a stage sits at 16-byte position c ^ swz(r) of
// row r's 64 bytes.
__device__ __forceinline__ int tiled_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// rot: 0 none, 1 Hadamard-32, 2 Kronecker (P x Q), 3 per-channel smoothing;
// FIT: fitted block exponents (offline weight quantization).
//
// Work split: every wave quantizes 64 blocks.  Row-major output: 64
// consecutive blocks in row-major block order.  Tiled output: the 4 blocks of
// one 128-element stage in 16 consecutive rows, so the wave's code stores are
// one contiguous KiB of the tiled layout.  Padding rows inside the last
// 16-row group load as zeros and store zero codes and scales; the 16-row
// groups past it are not written at all (no GEMM output depends on them).
template <bool BF16, int ROT, int P, int Q, bool FIT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a, int dense) {
  constexpr int CPB = BF16 ? 4 : 8;   // 16-byte chunks per 32-element block
  __shared__ u32x4 slab[kThreads / 64][64 * CPB];
  // the wave index is uniform: the per-wave address set-up (the division
  // below, the layout branches) runs on the scalar unit
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wid = blockIdx.x * (kThreads / 64) + wave;   // global wave index
  const uint32_t nblk = a.rows * a.nblk_row;
  const uint32_t nstage = a.nblk_row / 4;
  uint32_t wb0 = 0, rg = 0, st = 0;
  if (a.tiled) {
    rg = wid / nstage;
    st = wid - rg * nstage;
    if (rg * 16 >= a.rows) return;
  } else {
    wb0 = wid * 64;
    if (wb0 >= nblk) return;
  }
  // (row, block column) of local block bl of this wave; false if outside X
  auto locate = [&](int bl, uint32_t& row, uint32_t& col) -> bool {
    if (a.tiled) {
      row = rg * 16 + (bl >> 2);
      col = 4 * st + (bl & 3);
      return row < a.rows;
    }
    const uint32_t g = wb0 + bl;
    if (dense) {
      row = 0;
      col = g;   // row-contiguous blocks: g * 32 elements from x
    } else {
      row = g / a.nblk_row;
      col = g - row * a.nblk_row;
    }
    return g < nblk;
  };
  const int esz = BF16 ? 2 : 4;
  const uint8_t* x = static_cast<const uint8_t*>(a.x);

  // coalesced loads: instruction u covers chunks 64u .. 64u + 63 of the wave.
  // A wave whose blocks all lie inside X (every wave but the last) loads
  // without predicates; the edge wave loads zeros past the end.
  const bool all_in = a.tiled ? rg * 16 + 16 <= a.rows : wb0 + 64 <= nblk;
  u32x4 ld[CPB];
  if (all_in && a.tiled) {
    // tiled order: the wave's input is rows 16 rg .. 16 rg + 15, elements
    // 128 st .. 128 st + 127 of each, i.e. CPR 16-byte chunks per row; chunk
    // c = 64 u + lane sits in row c / CPR at byte 16 (c % CPR)
    constexpr int CPR = 4 * CPB;
    const int64_t rstride = a.ld_x * esz;
    const uint8_t* base = x + ((int64_t)(rg * 16) * a.ld_x + (int64_t)st * 128) * esz +
                          (lane / CPR) * rstride + (lane % CPR) * 16;
#pragma unroll
    for (int u = 0; u < CPB; ++u)
      ld[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + u * (64 / CPR) * rstride));
  } else if (all_in && dense) {
    // dense row-major rows: the wave's 64 blocks are one contiguous run
    const uint8_t* base = x + (int64_t)wb0 * 32 * esz + lane * 16;
#pragma unroll
    for (int u = 0; u < CPB; ++u) ld[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + u * 1024));
  } else if (all_in) {
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int c = 64 * u + lane;
      uint32_t row, col;
      locate(c / CPB, row, col);
      const int64_t off = ((int64_t)row * a.ld_x + (int64_t)col * 32) * esz;
      ld[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off + 16 * (c % CPB)));
    }
  } else {
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      const int c = 64 * u + lane;
      uint32_t row, col;
      if (locate(c / CPB, row, col)) {
        const int64_t off = ((int64_t)row * a.ld_x + (int64_t)col * 32) * esz;
        ld[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + off + 16 * (c % CPB)));
      } else {
        ld[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int u = 0; u < CPB; ++u) {
    const int c = 64 * u + lane;
    const int bl = c / CPB;
    slab[wave][bl * CPB + ((c % CPB) ^ slab_swz<CPB>(bl))] = ld[u];
  }
  // The slab is private to this wave and LDS operations of one wave complete
  // in order, so the reads below see the writes above without a barrier.
  uint32_t orow, ocol;
  const bool inside = locate(lane, orow, ocol);
  if (!a.tiled && !inside) return;
  u32x4 q4[CPB];
#pragma unroll
  for (int q = 0; q < CPB; ++q) q4[q] = slab[wave][lane * CPB + (q ^ slab_swz<CPB>(lane))];

  uint32_t w[4];
  uint32_t sbyte;
  if constexpr (BF16 && ROT == 0 && !FIT) {
    // no transform: amax and codes straight from the packed bf16 pairs
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) d[4 * i + j] = q4[i][j];
    sbyte = encode_block_bf16(d, w);
  } else {
    float v[32];
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_lo(q4[i][j]);
          v[8 * i + 2 * j + 1] = bf16_hi(q4[i][j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = __uint_as_float(q4[i][j]);
    }
    // smoothing factors of this block's 32 channels (block column within its row)
    const uint32_t kcol = (!a.tiled && dense) ? ocol % a.nblk_row : ocol;
    rotate_block<ROT, P, Q>(ROT == 3 ? a.fa + 32 * kcol : a.fa, a.fb, v);
    sbyte = encode_block_sel<FIT>(v, w);
  }
  if (a.tiled) {
    const uint32_t t = orow / kTileRows, r = orow % kTileRows, sg = ocol / 4, cb = ocol % 4;
    const uint64_t ts = (uint64_t)t * nstage + sg;   // (tile, stage) index
    uint4* dst = reinterpret_cast<uint4*>(a.codes + ts * (kTileRows * 64) + r * 64) + (cb ^ tiled_swz(r));
    *dst = make_uint4(w[0], w[1], w[2], w[3]);
    a.scales[ts * (kTileRows * 4) + r * 4 + cb] = static_cast<uint8_t>(sbyte);
  } else {
    const uint32_t gid = wb0 + lane;
    uint4* dst = reinterpret_cast<uint4*>(a.codes) + gid;
    *dst = make_uint4(w[0], w[1], w[2], w[3]);   // the GEMM reads these next: keep them cached
    a.scales[gid] = static_cast<uint8_t>(sbyte);
  }
}

// Few blocks with a Kronecker transform (decode-sized inputs, which fill a
// fraction of the chip): there the time is the latency of one lane's P*Q*(P+Q)
// dependent-chain FMAs, so each block is spread over Q lanes instead of one.
// Lane k of a block's group computes column k of the first stage, U[j][k] for
// every j, and then the outputs y[Q*i+k] of the second stage -- the same
// chains, in the same order, as the one-lane transform, so the values are
// identical.  The group then takes the block amax with a butterfly of max
// reductions, converts its P values at the block scale, merges the nibbles
// with OR butterflies, and its first lane stores the 16 code bytes and the
// scale byte.  Blocks are numbered row-major over the rows that the output
// layout holds (tiled: whole 16-row groups, padding rows from zero inputs).
template <bool BF16, int P, int Q>
__global__ __launch_bounds__(kThreads) void quantize_kron_lanes_kernel(QuantArgs a, uint32_t nblocks) {
  static_assert(P * Q == 32 && Q >= 2 && Q <= 32, "factor sizes");
  const int lane = threadIdx.x & 63;
  const int k = lane % Q;
  const uint32_t blk = (blockIdx.x * kThreads + threadIdx.x) / Q;
  const bool live = blk < nblocks;
  const uint32_t row = live ? blk / a.nblk_row : 0u;
  const uint32_t col = live ? blk - row * a.nblk_row : 0u;

  float v[32];
  if (live && row < a.rows) {
    const uint8_t* src = static_cast<const uint8_t*>(a.x) + ((int64_t)row * a.ld_x + (int64_t)col * 32) * (BF16 ? 2 : 4);
    if constexpr (BF16) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * c + 2 * j] = bf16_lo(q[j]);
          v[8 * c + 2 * j + 1] = bf16_hi(q[j]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * c + j] = __uint_as_float(q[j]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }

  // the block as the P x Q matrix Xm[j][l] = v[Q*j+l]; factors are uniform
  const float* fa = a.fa;
  const float* fb = a.fb;
  float u[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    float acc = fb[k * Q] * v[Q * j];
#pragma unroll
    for (int l = 1; l < Q; ++l) acc = __builtin_fmaf(fb[k * Q + l], v[Q * j + l], acc);
    u[j] = acc;
  }
  float y[P];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    float acc = fa[i * P] * u[0];
#pragma unroll
    for (int j = 1; j < P; ++j) acc = __builtin_fmaf(fa[i * P + j], u[j], acc);
    y[i] = acc;
    am = fmaxf(am, fabsf(acc));
  }
#pragma unroll
  for (int o = 1; o < Q; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
  const uint32_t sbyte = sbyte_of_amax(am);
  const float scale = scale_of(sbyte);

  // element Q*i+k goes to nibble (Q*i+k) % 8 of code dword (Q*i+k) / 8
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = Q * i + k;
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[i], 0.0f, scale, 0) & 0xFu;
    const uint32_t sh = 4u * (uint32_t)(e & 7);
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] |= (e >> 3) == d ? c << sh : 0u;
  }
#pragma unroll
  for (int o = 1; o < Q; o <<= 1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] |= (uint32_t)__shfl_xor((int)w[d], o);
  }
  if (!live || k != 0) return;
  if (a.tiled) {
    const uint32_t nstage = a.nblk_row / 4;
    const uint32_t t = row / kTileRows, r = row % kTileRows, sg = col / 4, cb = col % 4;
    const uint64_t ts = (uint64_t)t * nstage + sg;
    uint4* dst = reinterpret_cast<uint4*>(a.codes + ts * (kTileRows * 64) + r * 64) + (cb ^ tiled_swz(r));
    *dst = make_uint4(w[0], w[1], w[2], w[3]);
    a.scales[ts * (kTileRows * 4) + r * 4 + cb] = static_cast<uint8_t>(sbyte);
  } else {
    const uint64_t gid = (uint64_t)row * a.nblk_row + col;
    reinterpret_cast<uint4*>(a.codes)[gid] = make_uint4(w[0], w[1], w[2], w[3]);
    a.scales[gid] = static_cast<uint8_t>(sbyte);
  }
}

// Block counts up to this take the Q-lanes-per-block Kronecker kernel.
#ifndef MXFP4_KRON_LANES_MAX_BLOCKS
#define MXFP4_KRON_LANES_MAX_BLOCKS 16384
#endif
constexpr uint64_t kKronLanesMaxBlocks = MXFP4_KRON_LANES_MAX_BLOCKS;

template <bool BF16, int P, int Q>
void launch_kron_lanes(const QuantArgs& a, uint64_t blocks, hipStream_t s) {
  const dim3 grid((uint32_t)((blocks * Q + kThreads - 1) / kThreads)), block(kThreads);
  quantize_kron_lanes_kernel<BF16, P, Q><<<grid, block, 0, s>>>(a, (uint32_t)blocks);
}

template <bool BF16, bool FIT>
hipError_t dispatch(const QuantArgs& a, hipStream_t s) {
  const uint64_t rows = a.tiled ? (a.rows + 15) / 16 * 16 : a.rows;   // tiled: whole 16-row groups
  const uint64_t blocks = rows * a.nblk_row;   // 64 per wave
  const dim3 grid((uint32_t)((blocks + kThreads - 1) / kThreads)), block(kThreads);
  const int dense = a.ld_x == (int64_t)a.nblk_row * 32;
  if (a.rot == 0) {
    quantize_kernel<BF16, 0, 1, 32, FIT><<<grid, block, 0, s>>>(a, dense);
  } else if (a.rot == 1) {
    quantize_kernel<BF16, 1, 1, 32, FIT><<<grid, block, 0, s>>>(a, dense);
  } else if (a.rot == 3) {
    quantize_kernel<BF16, 3, 1, 32, FIT><<<grid, block, 0, s>>>(a, dense);
  } else if (!FIT && blocks <= kKronLanesMaxBlocks && a.p >= 1 && a.p <= 16) {
    switch (a.p) {
      case 1: launch_kron_lanes<BF16, 1, 32>(a, blocks, s); break;
      case 2: launch_kron_lanes<BF16, 2, 16>(a, blocks, s); break;
      case 4: launch_kron_lanes<BF16, 4, 8>(a, blocks, s); break;
      case 8: launch_kron_lanes<BF16, 8, 4>(a, blocks, s); break;
      case 16: launch_kron_lanes<BF16, 16, 2>(a, blocks, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.p) {
      case 1: quantize_kernel<BF16, 2, 1, 32, FIT><<<grid, block, 0, s>>>(a, dense); break;
      case 2: quantize_kernel<BF16, 2, 2, 16, FIT><<<grid, block, 0, s>>>(a, dense); break;
      case 4: quantize_kernel<BF16, 2, 4, 8, FIT><<<grid, block, 0, s>>>(a, dense); break;
      case 8: quantize_kernel<BF16, 2, 8, 4, FIT><<<grid, block, 0, s>>>(a, dense); break;
      case 16: quantize_kernel<BF16, 2, 16, 2, FIT><<<grid, block, 0, s>>>(a, dense); break;
      case 32: quantize_kernel<BF16, 2, 32, 1, FIT><<<grid, block, 0, s>>>(a, dense); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, bool bf16, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.fit) return bf16 ? dispatch<true, true>(a, s) : dispatch<false, true>(a, s);
  return bf16 ? dispatch<true, false>(a, s) : dispatch<false, false>(a, s);
}

}  // namespace mxfp4
