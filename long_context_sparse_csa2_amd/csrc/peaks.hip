// Measurement kernels behind the box-measured peaks that the benchmark
// reports beside the datasheet figures: a streaming read of a device buffer
// (the practical HBM read ceiling of a kernel) and a loop of dense bf16
// 32x32x16 MFMAs on register operands (the practical matrix ceiling).
// Neither is a step of the path.
#include "common.h"
#include "launch.h"
#include "csa2_peaks.h"

namespace csa2 {

constexpr int PK_THREADS = 256;

// Grid-stride read of n16 16-byte words, eight loads in flight per lane;
// the words are folded by xor and written only if the fold hits a constant
// no buffer of practical size produces, so the loads stay and nothing is
// written.
constexpr int PK_UNROLL = 8;

__global__ __launch_bounds__(PK_THREADS) void k_peak_read(const u32x4_t* __restrict__ p,
                                                         int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * PK_THREADS;
  int64_t i = (int64_t)blockIdx.x * PK_THREADS + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (PK_UNROLL - 1) * stride < n16; i += PK_UNROLL * stride) {
    u32x4_t v[PK_UNROLL];
#pragma unroll
    for (int u = 0; u < PK_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < PK_UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == 0x9E3779B9u && acc[0] == 0x7F4A7C15u) sink[blockIdx.x] = v;
}

// Four independent accumulator chains of 32x32x16 bf16 MFMAs per wave.
__global__ __launch_bounds__(PK_THREADS) void k_peak_mfma(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(float)((t + j) & 7);
    b[j] = (__bf16)(float)((t * 3 + j) & 5);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32_bf16(a, b, c0);
    c1 = mfma32_bf16(b, a, c1);
    c2 = mfma32_bf16(a, a, c2);
    c3 = mfma32_bf16(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (s == -1.f) sink[blockIdx.x] = s;                 // never: the sums are >= 0
}

}  // namespace csa2

extern "C" {

int csa2_peak_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0) return 1;
  hipLaunchKernelGGL(csa2::k_peak_read, dim3(4096), dim3(csa2::PK_THREADS), 0, (hipStream_t)stream,
                     (const u32x4_t*)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

double csa2_peak_mfma(int iters, float* sink, void* stream) {
  if (!sink || iters < 1) return -1.0;
  const int grid = 1024;                               // 4096 waves: four per SIMD
  hipLaunchKernelGGL(csa2::k_peak_mfma, dim3(grid), dim3(csa2::PK_THREADS), 0, (hipStream_t)stream,
                     iters, sink);
  if (hipGetLastError() != hipSuccess) return -1.0;
  const double waves = (double)grid * (csa2::PK_THREADS / 64);
  return waves * iters * 4.0 * (2.0 * 32 * 32 * 16);
}

}  // extern "C"
