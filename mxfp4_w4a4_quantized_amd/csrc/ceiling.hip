// Measurement kernels, not part of the MXFP4 path.
//
// mxfp4_ceiling_mfma: the rate at which this
// device sustains the block-scaled FP4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4,
// E2M1 operands, one E8M0 byte per 32-element block, as the large GEMM issues
// it) when every SIMD of every CU issues it back to back, with no memory
// traffic at all.  The dense FP4 peak assumes the peak engine clock; under
// this load the clock the device holds is lower, and this kernel measures
// what that leaves.  The benchmark reports it beside the GEMM's roofline.
//
// One workgroup of four waves per CU (one wave per SIMD, as the GEMM).  Each
// wave keeps 8 independent accumulators (no MFMA waits on another's result)
// and cycles through 4 A and 4 B operand registers filled with pseudo-random
// codes and per-MFMA scale bytes, so the operands toggle like real data.
//
// mxfp4_ceiling_stream: the HBM rate of a bare streaming kernel with the
// memory pattern of the quantizer and of the decode GEMM and no arithmetic:
// each wave reads `rk` KiB (one KiB per load instruction, 16 contiguous
// bytes per lane, non-temporal) and writes `wk` KiB (wk <= rk) the same way:
// with rk = 4 a wave's KiB are contiguous (the quantizer's pattern), with
// rk = 16 its loads are spread over the buffer (the decode GEMM's).
// Its time over the same byte counts is the practical ceiling of a kernel of
// that size: launch, ramp and drain included.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {   // 32-bit integer hash (xorshift-multiply)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256, 1) void mfma_loop(float* out, unsigned long long* cycles, int iters, uint32_t seed) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t base = seed * 0x9e3779b9u + (blockIdx.x * 256u + threadIdx.x) * 64u;
  v8i a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // FP4 operands use the first 4 registers
      a[s][i] = i < 4 ? (int)mix(base + 8 * s + i) : 0;
      b[s][i] = i < 4 ? (int)mix(base + 32 + 8 * s + i) : 0;
    }
  uint32_t sa[8], sb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {   // scale bytes 120..135 in all four byte lanes
    sa[j] = 0x78787878u + (mix(base + 100 + j) & 0x0f0f0f0fu);
    sb[j] = 0x78787878u + (mix(base + 200 + j) & 0x0f0f0f0fu);
  }
  v16f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j & 3], b[(j + u) & 3], acc[j], 4, 4, 0,
                                                                 (int)sa[j], 1, (int)sb[7 - j]);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();

  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[j][r];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
  if (lane == 0) cycles[blockIdx.x * 4 + wave] = (unsigned long long)(t1 - t0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// STRIDED: load i of wave w takes KiB i * waves + w, so every load
// instruction of the grid sweeps the buffer in step (the decode GEMM's waves
// read one KiB from each of several 16 KiB stage blocks); else the wave's
// rk KiB are contiguous (the quantizer's waves).  The store count is a
// template parameter so the loaded registers are indexed at compile time.
template <int RK, int WK, bool STRIDED>
__global__ __launch_bounds__(256) void stream_loop(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                    int64_t waves) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= waves) return;
  u32x4 v[RK];
#pragma unroll
  for (int i = 0; i < RK; ++i)
    v[i] = __builtin_nontemporal_load(src + (STRIDED ? (i * waves + wave) : (wave * RK + i)) * 64 + lane);
  u32x4* d = dst + wave * WK * 64 + lane;
#pragma unroll
  for (int i = 0; i < WK; ++i) {   // each store carries data of every load
    u32x4 x = v[i];
#pragma unroll
    for (int j = 0; j < RK; ++j)
      if (j != i) x ^= v[j];
    __builtin_nontemporal_store(x, d + 64 * i);
  }
  if constexpr (WK == 0) {   // keep the loads live: a store that never happens in practice
    u32x4 x = v[0];
#pragma unroll
    for (int j = 1; j < RK; ++j) x ^= v[j];
    if (x[0] == 0x9e3779b9u && x[1] == 0x7f4a7c15u && x[2] == 0x12345678u && x[3] == 0xdeadbeefu) dst[lane] = x;
  }
}

}  // namespace

// waves waves of 64 lanes (4 per workgroup); wave w reads rk KiB of src (KiB
// rk w .. rk w + rk - 1 for rk = 4 or 8, KiB i waves + w for i < 16 when rk =
// 16) and writes KiB wk w .. wk w + wk - 1 of dst ((rk, wk) one of (4, 0),
// (4, 1), (8, 0), (8, 2), (16, 0); dst at least 1 KiB when wk == 0).  src holds waves * rk
// KiB, dst waves * max(wk, 1) KiB, both 16-byte aligned device memory.
// Returns 0, or a HIP error code.
extern "C" __attribute__((visibility("default"))) int mxfp4_ceiling_stream(const void* src, void* dst, long long waves,
                                                                             int rk, int wk, void* stream) {
  if (src == nullptr || dst == nullptr || waves <= 0 || wk < 0 || wk > rk || ((uintptr_t)src % 16) != 0 ||
      ((uintptr_t)dst % 16) != 0)
    return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* a = static_cast<const u32x4*>(src);
  u32x4* b = static_cast<u32x4*>(dst);
  if (rk == 4 && wk == 0) stream_loop<4, 0, false><<<grid, block, 0, s>>>(a, b, waves);
  else if (rk == 4 && wk == 1) stream_loop<4, 1, false><<<grid, block, 0, s>>>(a, b, waves);
  else if (rk == 8 && wk == 0) stream_loop<8, 0, false><<<grid, block, 0, s>>>(a, b, waves);
  else if (rk == 8 && wk == 2) stream_loop<8, 2, false><<<grid, block, 0, s>>>(a, b, waves);
  else if (rk == 16 && wk == 0) stream_loop<16, 0, true><<<grid, block, 0, s>>>(a, b, waves);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// blocks workgroups (use the CU count), iters rounds of 8 MFMAs per wave (a
// multiple of 4).
// out: blocks * 256 floats, cycles: blocks * 4 counters (device memory); the
// launch goes to `stream`.  Returns 0, or the HIP error code of the launch.
extern "C" __attribute__((visibility("default"))) int mxfp4_ceiling_mfma(int blocks, int iters, float* out,
                                                                           unsigned long long* cycles, void* stream) {
  if (blocks <= 0 || iters <= 0 || iters % 4 != 0 || out == nullptr || cycles == nullptr)
    return (int)hipErrorInvalidValue;
  mfma_loop<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(out, cycles, iters, 12345u);
  return (int)hipGetLastError();
}
