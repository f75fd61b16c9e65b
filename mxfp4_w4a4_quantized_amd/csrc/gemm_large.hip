// Large-tile MXFP4 x MXFP4 GEMM for gfx950 on v_mfma_scale_f32_32x32x64_f8f6f4
// (both operands E2M1: cbsz = blgp = 4).
//
// Y[m][n] = sum_k a_hat[m][k] * b_hat[n][k], A (activations) and B (weights)
// K-major packed E2M1 with one E8M0 byte per 32-element block, read directly
// by the MFMA (no dequantize pass; "AMD Quark delivers MXFP4 quantization for
// FLUX.1-dev on Instinct MI350 with 1.92x speedup", sections "MXFP4
// quantization for diffusion models" and "What is MXFP4 and why does it
// eliminate dequantization overhead?").  fp32 accumulation, fp32 or bf16
// output.
//
// MFMA operand layout with FP4 operands (checked on the device): lane l
// supplies row l % 32 of its operand and the 32 K elements of block l / 32 as
// 16 packed bytes (low nibble first) -- 16 consecutive bytes of a K-major
// packed row -- plus one E8M0 byte for that block, picked by op_sel from a
// 32-bit register.  Accumulator register r of lane l holds
// D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].
//
// Design (one workgroup of 4 waves per CU, persistent over output tiles):
//  * Output tile 256 (N, weight rows) x 256 (M, activation rows); each wave
//    owns a 128 x 128 quadrant as 4 x 4 MFMA fragments (256 fp32
//    accumulators per lane).  The weight tile is the MFMA's first operand,
//    so each lane ends with runs of 4 consecutive output columns of one row.
//  * K advances in stages of 128 elements: per row 64 code bytes and one
//    32-bit word of 4 scale bytes.  Stages go global -> LDS with direct LDS
//    loads (global_load_lds_dwordx4 for codes, _dword for scales) into a ring
//    of NBUF buffers, NBUF - 1 stages ahead of the MFMAs, with one barrier
//    per stage.  The ring runs across tile boundaries, so the next tile's
//    first stages load during the current tile's last MFMAs and epilogue.
//  * A stage feeds two MFMA sub-steps; lane group g = l / 32 takes blocks
//    2g and 2g + 1 of the stage (sub-steps s = 0, 1), so its scale register
//    is the row's scale word shifted right by 16 g and op_sel = s.  Both
//    operands use the same block assignment, so every product pairs the
//    right blocks.
//  * 16-byte chunks of a 64-byte LDS row are XOR-swizzled by
//    ((row >> 1) ^ (row >> 2)) & 3, so every 16-lane phase of a fragment's
//    ds_read_b128 hits 16 distinct 16-byte bank groups of the 64-bank LDS.
//  * Fragments are double-buffered in registers: the second sub-step's
//    fragments load while the first sub-step's MFMAs run, and the next
//    stage's scales and first fragments load while the second sub-step's
//    MFMAs run.  The stage's barrier therefore sits before its first
//    sub-step, where it also certifies the next stage's arrival.
//  * Tiles are ordered in groups of 4 M-tiles (N fastest within a group),
//    and workgroup b, which the dispatcher places on XCD b % 8, takes logical
//    tiles so that the 32 workgroups of one XCD work on one compact 4 x 8
//    block of tiles at a time and share its operand panels in that XCD's L2.
//  * Row-major operands: rows beyond M or N are clamped to a valid row (never
//    stored).  Tiled operands (the library's GEMM-native layout) hold each
//    stage of each 256-row tile as the exact LDS image, so every load is one
//    contiguous KiB of codes or 256 bytes of scales; their padding rows are
//    zero.  K must be a multiple of 128 (the host routes other row-major
//    shapes to the general kernel).
#include "internal.h"

#include <atomic>

#ifndef MXFP4_GEMM_WN
#define MXFP4_GEMM_WN 2
#define MXFP4_GEMM_WM 2
#endif

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 256;                      // weight rows per tile
constexpr int BM = 256;                      // activation rows per tile
constexpr int KS = 128;                      // K elements per stage
constexpr int RB = KS / 2;                   // code bytes per row per stage
constexpr int ROWS = BN + BM;                // rows per stage: W then X
constexpr int NBUF = 4;                      // LDS ring depth
constexpr int CODE_BYTES = ROWS * RB;        // 32 KiB
constexpr int STAGE_BYTES = CODE_BYTES + ROWS * 4;
constexpr int GROUP_M = 4;

static_assert(NBUF * STAGE_BYTES <= 160 * 1024, "LDS ring exceeds 160 KiB");

// Chunk swizzle: rows r and r + 4, r + 8, r + 12 (one 16-lane phase of a
// ds_read_b128 on the 64-bank LDS) and rows r, r + 2, r + 4, r + 6 (one
// 8-lane phase of a 32-bank LDS) all land in distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

template <int S>
__device__ __forceinline__ v16f mma(const u32x4& a, const u32x4& b, const v16f& c, uint32_t sa,
                                    uint32_t sb) {
  const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, S, (int)sa, S, (int)sb);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// One accumulator read straight from its AGPR.  The epilogues read their
// accumulators through this, one fragment at a time: with plain reads the
// register allocator copied all 256 out of the AGPRs at the loop exit in the
// MXFP4-output epilogue (which spilled), and paired each read with its pack
// through two temporaries in the bf16 one.
__device__ __forceinline__ float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// Zeroed accumulators for each tile.  With a plain 0.f the compiler
// materialized the 256 zeros of a tile twice (once for a K loop that might
// not run), 512 register writes per wave and tile.  An opaque zero cannot be
// rematerialized: acc_zero() is one v_accvgpr_write (the fp32-output kernel),
// acc_zero_mfma() one MFMA of zero codes with a zero accumulator input that
// clears a whole fragment's 16 registers on the matrix pipe, which is idle
// between tiles (the bf16 and MXFP4-output kernels, whose epilogues read every
// accumulator through acc_read).  Both compiled without spills; zeros from
// the MFMA builtin, or a first K stage started from the MFMA's zero operand,
// made the compiler copy or spill the accumulators.
__device__ __forceinline__ float acc_zero() {
  float r;
  asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(r));
  return r;
}

// The compiler places no wait states before an MFMA it cannot see: the nop
// separates it from a VALU write of its operand registers just before it.
__device__ __forceinline__ void acc_zero_mfma(v16f& acc, const u32x4& zero_codes) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %1, 0 cbsz:4 blgp:4" : "=a"(acc) : "v"(zero_codes));
}

__device__ __forceinline__ void tile_coords(int L, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GROUP_M * tiles_n;
  const int grp = L / per_group;
  const int first_m = grp * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int r = L - grp * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// Wait until at most `pending` stages of this wave's direct LDS loads are
// still in flight (vector memory loads of one wave complete in order, so a
// count that only covers the later stages' loads is enough even with stores
// outstanding).
template <int PENDING, int LOADS_PER_STAGE>
__device__ __forceinline__ void wait_stages() {
  // s_waitcnt simm16 on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  constexpr int n = PENDING * LOADS_PER_STAGE;
  static_assert(n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Scheduling pattern of one MFMA sub-step: MF MFMAs; RD LDS reads issued two
// per MFMA from the second MFMA on (they feed the next sub-step); VM global
// loads spread evenly over the MFMAs after the reads, so that the four waves'
// loads reach the texture unit at a steady rate.
template <int MF, int RD, int VM, int I = 0, int RDL = RD, int VML = VM>
__device__ __forceinline__ void sched_substep() {
  if constexpr (I < MF) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // 1 MFMA
    constexpr int rd = (I >= 1 && RDL > 0) ? (RDL >= 2 ? 2 : 1) : 0;
    if constexpr (rd > 0) __builtin_amdgcn_sched_group_barrier(0x100, rd, 0);   // LDS reads
    constexpr int from = (RD + 1) / 2 + 1;
    constexpr int span = MF - from > 0 ? MF - from : 1;
    constexpr int vm = (I >= from) ? ((I - from + 1) * VM) / span - ((I - from) * VM) / span : 0;
    constexpr int vmc = vm < VML ? vm : VML;
    if constexpr (vmc > 0) __builtin_amdgcn_sched_group_barrier(0x010, vmc, 0);  // global loads
    sched_substep<MF, RD, VM, I + 1, RDL - rd, VML - vmc>();
  } else {
    if constexpr (RDL > 0) __builtin_amdgcn_sched_group_barrier(0x100, RDL, 0);
    if constexpr (VML > 0) __builtin_amdgcn_sched_group_barrier(0x010, VML, 0);
  }
}

// WN x WM waves; each wave owns a (BN / WN) x (BM / WM) block of the tile as
// FN x FM fragments of 32 x 32.
constexpr int WN = MXFP4_GEMM_WN, WM = MXFP4_GEMM_WM;
constexpr int NT = 64 * WN * WM;

// OUT: 0 fp32 Y, 1 bf16 Y, 2 MXFP4 Y (requantized per 32-block along N).
template <int OUT>
__global__ __launch_bounds__(NT, 1) void gemm_large_kernel(GemmArgs g, int tiles_m, int tiles_n, int grid,
                                                           int xcd_remap, int y_vec) {
  constexpr int NW = WN * WM;
  constexpr int FN = BN / WN / 32, FM = BM / WM / 32;
  constexpr int CODE_LOADS = CODE_BYTES / 1024 / NW;   // per wave, 16 B per lane
  constexpr int SCALE_LOADS = ROWS * 4 / 256 / NW;     // per wave, 4 B per lane
  constexpr int LPS = CODE_LOADS + SCALE_LOADS;
  constexpr int CODE_LOADS_B = CODE_LOADS / 2;         // issued during sub-step 0
  static_assert(CODE_LOADS >= 1 && SCALE_LOADS >= 1, "wave count");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * STAGE_BYTES];

  const int ntiles = tiles_m * tiles_n;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int slot = xcd_remap ? (b & 7) * (grid >> 3) + (b >> 3) : b;
  if (slot >= ntiles) return;
  const int nk = g.k / KS;
  const int total = ((ntiles - slot + grid - 1) / grid) * nk;
  const uint32_t kbytes = (uint32_t)g.k / 2, kblocks = (uint32_t)g.k / 32;
  // output rows start 16-byte aligned: the staged epilogue's 16-byte stores
  constexpr bool BF16OUT = OUT == 1;
  const bool y_st = OUT == 2 || (((uintptr_t)g.y % 16) == 0 && ((g.ld_y * (BF16OUT ? 2 : 4)) % 16) == 0);

  // ---- direct LDS load plan: the first half of the waves loads weight rows,
  // the second half activation rows; wave w fills stage rows
  // [16 * CODE_LOADS * w, 16 * CODE_LOADS * (w + 1)).
  const bool w_side = wave < NW / 2;
  const uint8_t* cbase = w_side ? g.b_codes : g.a_codes;
  const uint8_t* sbase = w_side ? g.b_scales : g.a_scales;
  const int lim = (w_side ? g.n : g.m) - 1;
  const int part = wave % (NW / 2);
  uint32_t coff[CODE_LOADS], soff[SCALE_LOADS];
  // Row-major operands: each load takes 16 rows x 64 bytes (rows clamped to
  // the last valid row).  Tiled operands: each load takes one contiguous KiB
  // (codes) or 256 bytes (scales) that already hold the LDS image.
  const bool tiled = g.tiled;
  const uint32_t nstage = (uint32_t)nk;
  auto plan = [&](int j) {   // j-th tile of this workgroup
    int tm, tn;
    tile_coords(j * grid + slot, tiles_m, tiles_n, tm, tn);
    const int tile = w_side ? tn : tm;
    const int r0 = tile * (w_side ? BN : BM);
#pragma unroll
    for (int i = 0; i < CODE_LOADS; ++i) {
      const int rgp = CODE_LOADS * part + i;                   // 16-row group within this side
      if (tiled) {
        coff[i] = (uint32_t)tile * nstage * (16 * 1024) + rgp * 1024 + lane * 16;
      } else {
        const int row = 16 * rgp + (lane >> 2);
        const uint32_t grow = (uint32_t)min(r0 + row, lim);
        coff[i] = grow * kbytes + 16u * (uint32_t)((lane & 3) ^ swz(row));
      }
    }
#pragma unroll
    for (int i = 0; i < SCALE_LOADS; ++i) {
      const int row = 64 * (SCALE_LOADS * part + i) + lane;
      soff[i] = tiled ? (uint32_t)tile * nstage * 1024 + row * 4 : (uint32_t)min(r0 + row, lim) * kblocks;
    }
  };
  const uint32_t cstride = tiled ? 16 * 1024 : RB, sstride = tiled ? 1024 : 4;   // bytes per stage
  // Issue state: tile ij of this workgroup, stage ikt within it, ring slot
  // ibuf.  The loads of one stage are issued in pieces spread through the
  // MFMA stream, and advance() moves to the next stage.
  int ij = 0, ikt = 0, ibuf = 0;
  plan(0);
  auto issue_codes = [&](int i0, int i1) {
    uint8_t* dst = lds + ibuf * STAGE_BYTES;
    const uint8_t* cb = cbase + ikt * cstride;
#pragma unroll
    for (int i = i0; i < i1; ++i)
      __builtin_amdgcn_global_load_lds(cb + coff[i], dst + (CODE_LOADS * wave + i) * 1024, 16, 0, 0);
  };
  auto issue_scales = [&]() {
    uint8_t* dst = lds + ibuf * STAGE_BYTES;
    const uint8_t* sb = sbase + ikt * sstride;
#pragma unroll
    for (int i = 0; i < SCALE_LOADS; ++i)
      __builtin_amdgcn_global_load_lds(sb + soff[i],
                                       dst + CODE_BYTES + (64 * (SCALE_LOADS * wave + i)) * 4, 4, 0, 0);
  };
  auto advance = [&]() {
    ibuf = ibuf + 1 == NBUF ? 0 : ibuf + 1;
    if (++ikt == nk) {
      ikt = 0;
      if ((++ij) * nk < total) plan(ij);
    }
  };

  const int wn = wave % WN, wm = wave / WN;
  const int lr = lane & 31, lg = lane >> 5;
  // stage rows of this lane's fragments
  int wrow[FN], xrow[FM];
#pragma unroll
  for (int f = 0; f < FN; ++f) wrow[f] = wn * (BN / WN) + 32 * f + lr;
#pragma unroll
  for (int f = 0; f < FM; ++f) xrow[f] = BN + wm * (BM / WM) + 32 * f + lr;
  // Lane group g takes blocks 2g, 2g + 1 of a stage: a 16-bit load of the
  // row's scale bytes 2g, 2g + 1 leaves the sub-step s byte at op_sel = s.
  auto load_scales = [&](const uint8_t* sbuf, uint32_t (&sw)[FN], uint32_t (&sx)[FM]) {
#pragma unroll
    for (int f = 0; f < FN; ++f)
      sw[f] = *reinterpret_cast<const uint16_t*>(sbuf + CODE_BYTES + 4 * wrow[f] + 2 * lg);
#pragma unroll
    for (int f = 0; f < FM; ++f)
      sx[f] = *reinterpret_cast<const uint16_t*>(sbuf + CODE_BYTES + 4 * xrow[f] + 2 * lg);
  };
  auto load_frags = [&](const uint8_t* sbuf, int s, u32x4 (&wf)[FN], u32x4 (&xf)[FM]) {
    const int c = 2 * lg + s;
#pragma unroll
    for (int f = 0; f < FN; ++f)
      wf[f] = *reinterpret_cast<const u32x4*>(sbuf + wrow[f] * RB + 16 * (c ^ swz(wrow[f])));
#pragma unroll
    for (int f = 0; f < FM; ++f)
      xf[f] = *reinterpret_cast<const u32x4*>(sbuf + xrow[f] * RB + 16 * (c ^ swz(xrow[f])));
  };

  // The ring always has NBUF - 1 stages in flight: one stage is issued per
  // computed stage, past the end too (those re-read rows of the last tile into
  // a free slot and are never used), so every wait count is a constant.
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p) {
    if (p > 0) advance();
    issue_codes(0, CODE_LOADS);
    issue_scales();
  }

  // stage 0: wait for it, then load its scales and first fragments
  wait_stages<NBUF - 2, LPS>();
  __builtin_amdgcn_s_barrier();
  uint32_t sw[FN], sx[FM];
  u32x4 wa[FN], xa[FM];
  load_scales(lds, sw, sx);
  load_frags(lds, 0, wa, xa);

  constexpr int NRD = FN + FM;                  // fragment reads per sub-step
  int cbuf = 0;   // ring slot of the stage being computed
  u32x4 zero_codes;
  {
    uint32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    zero_codes = u32x4{z, z, z, z};
  }
  // bf16 and MXFP4 output: each fragment is cleared in the epilogue right
  // after its accumulators are read, so the clearing MFMAs overlap the
  // epilogue's other work (bit-identical, 1-2% faster than clearing at the
  // top of each tile); the fp32-output kernel writes its zeros at the top
  v16f acc[FN][FM];
  if constexpr (OUT != 0) {
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int c = 0; c < FM; ++c) acc_zero_mfma(acc[a][c], zero_codes);
  }
  for (int j = 0; j * nk < total; ++j) {
    if constexpr (OUT == 0) {
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int c = 0; c < FM; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[a][c][r] = acc_zero();
    } else if constexpr (OUT == 1 && !(WN == 2 && WM == 2)) {
      // other wave layouts (MXFP4_GEMM_WN / _WM) take the direct-store
      // epilogue, which does not clear: clear here
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int c = 0; c < FM; ++c) acc_zero_mfma(acc[a][c], zero_codes);
    }
    // the compiler does not see these clears (inline asm): wait states before
    // the K loop's MFMAs take them as their accumulator input
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    for (int kt = 0; kt < nk; ++kt) {
      advance();   // to stage it + NBUF - 1 (its branch stays out of the MFMA block)
      // Stage it + 1 is loaded once this wave's loads of it are done and every
      // wave has passed the barrier.  The barrier also guarantees that all
      // waves have finished reading stage it - 1, whose slot this iteration's
      // loads overwrite.  No fence: a release fence on LDS would also wait for
      // the loads still in flight.
      wait_stages<NBUF - 3, LPS>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);

      const uint8_t* sbuf = lds + cbuf * STAGE_BYTES;
      cbuf = cbuf + 1 == NBUF ? 0 : cbuf + 1;
      const uint8_t* nbuf = lds + cbuf * STAGE_BYTES;

      // sub-step 0 MFMAs, interleaved with the sub-step 1 reads and part of
      // the loads of stage it + NBUF - 1
      u32x4 wb[FN], xb[FM];
      load_frags(sbuf, 1, wb, xb);
      issue_codes(0, CODE_LOADS_B);
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int bb = 0; bb < FM; ++bb) acc[a][bb] = mma<0>(wa[a], xa[bb], acc[a][bb], sw[a], sx[bb]);
      sched_substep<FN * FM, NRD, CODE_LOADS_B>();

      // sub-step 1 MFMAs, interleaved with the next stage's scale and
      // sub-step 0 reads (after the last stage these read a slot that is
      // never used) and the rest of the loads
      uint32_t sw1[FN], sx1[FM];
#pragma unroll
      for (int f = 0; f < FN; ++f) sw1[f] = sw[f];
#pragma unroll
      for (int f = 0; f < FM; ++f) sx1[f] = sx[f];
      load_scales(nbuf, sw, sx);
      load_frags(nbuf, 0, wa, xa);
      issue_codes(CODE_LOADS_B, CODE_LOADS);
      issue_scales();
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int bb = 0; bb < FM; ++bb) acc[a][bb] = mma<1>(wb[a], xb[bb], acc[a][bb], sw1[a], sx1[bb]);
      sched_substep<FN * FM, 2 * NRD, LPS - CODE_LOADS_B>();
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- epilogue of this workgroup's j-th tile
    int tm, tn;
    tile_coords(j * grid + slot, tiles_m, tiles_n, tm, tn);
    if constexpr (OUT == 2) {
      // MXFP4 output, straight from the accumulators.  Fragment a of a wave
      // covers one 32-block along N for each of its 32 rows: lane l (row
      // l % 32, lane group g = l / 32) holds the runs n = 8 t + 4 g .. + 3,
      // t = 0..3, so the block's other half is in lane l ^ 32.  Block amax:
      // the lane's 16 values, then the partner's (exact); the E8M0 rule and
      // the E2M1 converter as in the quantizer.  One 32-bit exchange then
      // gives lane group 0 the block's code bytes 0..7 and group 1 bytes
      // 8..15, stored as 8 contiguous bytes per lane.
      // the wave's 128 columns start on a 128-column (tiled stage) boundary:
      // fragment a is block a of that stage, at chunk a ^ swz(row) (tiled)
      // or 16 a bytes further along the row (row-major)
      const int nw0 = tn * BN + wn * (BN / WN);
#pragma unroll
      for (int bb = 0; bb < FM; ++bb) {
        const int m = tm * BM + wm * (BM / WM) + 32 * bb + lr;
        uint8_t* cbase;
        uint8_t* sbase;
        int swr = 0;
        if (g.q_tiled) {
          const uint32_t r8 = (uint32_t)m & 255u;
          const uint64_t ts = (uint64_t)((uint32_t)m >> 8) * ((uint32_t)g.n >> 7) + ((uint32_t)nw0 >> 7);
          cbase = g.q_codes + ts * 16384 + r8 * 64;
          sbase = g.q_scales + ts * 1024 + r8 * 4;
          swr = swz((int)r8);
        } else {
          cbase = g.q_codes + (int64_t)m * (g.n >> 1) + (nw0 >> 1);
          sbase = g.q_scales + (int64_t)m * (g.n >> 5) + (nw0 >> 5);
        }
        const bool row_ok = m < g.m;
#pragma unroll
        for (int a = 0; a < FN; ++a) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = acc_read(acc[a][bb][r]);
          acc_zero_mfma(acc[a][bb], zero_codes);
          float am = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) am = fmaxf(am, fabsf(v[r]));
          am = fmaxf(am, __shfl_xor(am, 32));
          const uint32_t ef = __float_as_uint(am) >> 23;
          const uint32_t sb = ef > 2u ? ef - 2u : 0u;
          const float sc = __uint_as_float(sb ? sb << 23 : 0x00400000u);
          uint32_t w0 = 0, w1 = 0;   // runs t = 0, 1 and t = 2, 3: two code bytes per run
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[0], v[1], sc, 0);
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[2], v[3], sc, 1);
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[4], v[5], sc, 2);
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[6], v[7], sc, 3);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[8], v[9], sc, 0);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[10], v[11], sc, 1);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[12], v[13], sc, 2);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[14], v[15], sc, 3);
          // group 0 keeps w0 (bytes 0-1, 4-5) and takes the partner's w0
          // (bytes 2-3, 6-7); group 1 keeps w1 (bytes 10-11, 14-15) and
          // takes the partner's w1 (bytes 8-9, 12-13)
          const uint32_t recv = (uint32_t)__shfl_xor((int)(lg ? w0 : w1), 32);
          const uint32_t lo = lg ? recv : w0, hi = lg ? w1 : recv;
          const uint32_t d0 = (lo & 0xFFFFu) | (hi << 16), d1 = (lo >> 16) | (hi & 0xFFFF0000u);
          if (row_ok && nw0 + 32 * a < g.n) {
            const int chunk = g.q_tiled ? (a ^ swr) : a;
            *reinterpret_cast<uint2*>(cbase + 16 * chunk + 8 * lg) = make_uint2(d0, d1);
            if (lg == 0) sbase[a] = (uint8_t)sb;
          }
          // one fragment at a time: keeps the accumulator reads from being
          // hoisted together (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      continue;
    }
    if constexpr (WN == 2 && WM == 2) {
      // Stage each wave's 128 x 128 output block through the ring slot of
      // the stage just computed (free until the next issue, which follows the
      // next barrier), 32 rows x 256 bytes at a time in a padded 32 x
      // 272-byte area (4 bf16 or 2 fp32 fragments per pass), then store 4
      // full 256-byte rows per instruction (16 bytes per lane) instead of
      // short pieces of 32 rows.  Edge tiles and output rows that do not
      // start 16-byte aligned take the same staging with bounds-checked
      // stores, so there is one epilogue path: with two, the compiler copied
      // the accumulators to move their clearing into the epilogue.  bf16:
      // each fragment is cleared right after it is read.
      {
        const bool full = y_st && (tm + 1) * BM <= g.m && (tn + 1) * BN <= g.n;
        constexpr int PITCH = 272;
        constexpr int ESZ = BF16OUT ? 2 : 4;
        constexpr int FPP = 256 / (32 * ESZ);   // fragments per pass
        const int lslot = cbuf == 0 ? NBUF - 1 : cbuf - 1;
        uint8_t* tb = lds + lslot * STAGE_BYTES + wave * (32 * PITCH);
        __builtin_amdgcn_s_barrier();   // every wave is done reading that slot
#pragma unroll
        for (int bb = 0; bb < FM; ++bb) {
#pragma unroll
          for (int a0 = 0; a0 < FN; a0 += FPP) {
#pragma unroll
            for (int a = a0; a < a0 + FPP; ++a) {
              // bf16: the fragment's 16 accumulators first, then the packs
              // (plain reads went through two temporaries, one pair at a time)
              float v[16];
              if constexpr (BF16OUT) {
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = acc_read(acc[a][bb][r]);
                acc_zero_mfma(acc[a][bb], zero_codes);
              }
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                uint8_t* dst = tb + lr * PITCH + ((a - a0) * 32 + 8 * t + 4 * lg) * ESZ;
                if constexpr (BF16OUT) {
                  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(v[4 * t], v[4 * t + 1]),
                                                              pack_bf16(v[4 * t + 2], v[4 * t + 3]));
                } else {
                  *reinterpret_cast<float4*>(dst) = make_float4(acc[a][bb][4 * t], acc[a][bb][4 * t + 1],
                                                                acc[a][bb][4 * t + 2], acc[a][bb][4 * t + 3]);
                }
              }
            }
            // the area is private to this wave: its LDS writes land before its reads
            const int m0 = tm * BM + wm * (BM / WM) + 32 * bb;
            const int64_t n0 = tn * BN + wn * (BN / WN) + a0 * 32 + (lane & 15) * (16 / ESZ);
            if (full) {
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const int row = 4 * r + (lane >> 4);
                const uint4 v = *reinterpret_cast<const uint4*>(tb + row * PITCH + (lane & 15) * 16);
                // non-temporal: Y streams out without displacing the operand
                // panels the XCD's other workgroups still read from L2
                __builtin_nontemporal_store(
                    u32x4{v.x, v.y, v.z, v.w},
                    reinterpret_cast<u32x4*>(static_cast<uint8_t*>(g.y) + ((int64_t)(m0 + row) * g.ld_y + n0) * ESZ));
              }
            } else {
              // edge tiles and unaligned rows: bounds-checked stores of the same staged rows
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const int row = 4 * r + (lane >> 4);
                const uint4 v = *reinterpret_cast<const uint4*>(tb + row * PITCH + (lane & 15) * 16);
                if (m0 + row < g.m) {
                  uint8_t* yp = static_cast<uint8_t*>(g.y) + ((int64_t)(m0 + row) * g.ld_y + n0) * ESZ;
                  if (y_st && n0 + 16 / ESZ <= g.n) {
                    *reinterpret_cast<uint4*>(yp) = v;
                  } else {
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 16 / ESZ; ++e) {
                      if (n0 + e < g.n) {
                        if constexpr (ESZ == 2)
                          reinterpret_cast<uint16_t*>(yp)[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                        else
                          reinterpret_cast<uint32_t*>(yp)[e] = w4[e];
                      }
                    }
                  }
                }
              }
            }
          }
        }
        continue;
      }
    }
    if constexpr (OUT != 2 && !(WN == 2 && WM == 2)) {
#pragma unroll
    for (int bb = 0; bb < FM; ++bb) {
      const int m = tm * BM + wm * (BM / WM) + 32 * bb + lr;
      if (m >= g.m) continue;
#pragma unroll
      for (int a = 0; a < FN; ++a) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int n = tn * BN + wn * (BN / WN) + 32 * a + 8 * t + 4 * lg;
          float v0, v1, v2, v3;
          if constexpr (BF16OUT) {   // every bf16 read goes through acc_read (above)
            v0 = acc_read(acc[a][bb][4 * t]), v1 = acc_read(acc[a][bb][4 * t + 1]);
            v2 = acc_read(acc[a][bb][4 * t + 2]), v3 = acc_read(acc[a][bb][4 * t + 3]);
          } else {
            v0 = acc[a][bb][4 * t], v1 = acc[a][bb][4 * t + 1];
            v2 = acc[a][bb][4 * t + 2], v3 = acc[a][bb][4 * t + 3];
          }
          if constexpr (BF16OUT) {
            uint16_t* yp = static_cast<uint16_t*>(g.y) + (int64_t)m * g.ld_y + n;
            const uint32_t lo = pack_bf16(v0, v1), hi = pack_bf16(v2, v3);
            if (y_vec && n + 3 < g.n) {
              *reinterpret_cast<uint2*>(yp) = make_uint2(lo, hi);
            } else {
              if (n < g.n) yp[0] = (uint16_t)lo;
              if (n + 1 < g.n) yp[1] = (uint16_t)(lo >> 16);
              if (n + 2 < g.n) yp[2] = (uint16_t)hi;
              if (n + 3 < g.n) yp[3] = (uint16_t)(hi >> 16);
            }
          } else {
            float* yp = static_cast<float*>(g.y) + (int64_t)m * g.ld_y + n;
            if (y_vec && n + 3 < g.n) {
              *reinterpret_cast<float4*>(yp) = make_float4(v0, v1, v2, v3);
            } else {
              if (n < g.n) yp[0] = v0;
              if (n + 1 < g.n) yp[1] = v1;
              if (n + 2 < g.n) yp[2] = v2;
              if (n + 3 < g.n) yp[3] = v3;
            }
          }
        }
      }
    }
    }
  }
  // no direct LDS load may still be writing when the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

// CU count of the current device, cached per device.  Calls may come from
// several host threads at once: the cache slots are atomics (every writer
// stores the same value).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool gemm_large_supported(const GemmArgs& g) {
  const int64_t m = (g.m + BM - 1) / BM * BM, n = (g.n + BN - 1) / BN * BN;   // padded rows
  return (g.k % KS) == 0 && ((uintptr_t)g.a_scales % 4) == 0 && ((uintptr_t)g.b_scales % 4) == 0 &&
         m * (g.k / 2) < (int64_t(1) << 32) && n * (g.k / 2) < (int64_t(1) << 32) &&
         (!g.q_out || (g.n % (g.q_tiled ? 128 : 32)) == 0);
}

hipError_t launch_gemm_large(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (g.m + BM - 1) / BM, tiles_n = (g.n + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int cus = cu_count();
  int grid = ntiles < cus ? ntiles : cus;
  if (ntiles > cus) {
    // The rounds of tiles that one workgroup per CU needs, spread over the
    // fewest workgroups (a multiple of 8, one per XCD in turn) that still
    // take no more rounds, so that no round runs part-empty.  The chip runs
    // this kernel at its power limit, so a round on fewer CUs takes less
    // time: the 672 tiles of 3584 x 3072 -> 12288 take 73.3 us on 224
    // workgroups (3 full rounds) against 79.1 us on 256 (2.625 rounds).
    const int rounds = (ntiles + cus - 1) / cus;
    const int even = ((ntiles + rounds - 1) / rounds + 7) / 8 * 8;
    if (even < grid) grid = even;
  }
  const int xcd_remap = (grid % 8) == 0;
  const size_t ybytes = g.y_bf16 ? 2 : 4;
  const int y_vec = (((uintptr_t)g.y) % (4 * ybytes) == 0) && (g.ld_y % 4 == 0);
  if (g.q_out)
    gemm_large_kernel<2><<<grid, NT, 0, s>>>(g, tiles_m, tiles_n, grid, xcd_remap, y_vec);
  else if (g.y_bf16)
    gemm_large_kernel<1><<<grid, NT, 0, s>>>(g, tiles_m, tiles_n, grid, xcd_remap, y_vec);
  else
    gemm_large_kernel<0><<<grid, NT, 0, s>>>(g, tiles_m, tiles_n, grid, xcd_remap, y_vec);
  return hipGetLastError();
}

}  // namespace mxfp4
