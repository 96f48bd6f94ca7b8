// Optional checks of device data (indices) for debugging callers: enabled by
// CSA2_CHECK=1 in the environment, off otherwise.  Each check counts the
// out-of-range values of an int32 array into a per-device counter that the
// host reads back after synchronising the stream, so a checked call is not
// asynchronous and cannot be captured in a HIP graph.
#include "common.h"
#include "launch.h"

namespace csa2 {

__device__ unsigned int g_bad_count;     // out-of-range values seen by the last check

// a[r][c] for r < rows, c < min(len[r], ncols) (len NULL: ncols) must lie in
// [lo, hi).
__global__ __launch_bounds__(256) void k_check_range(const int32_t* __restrict__ a, int64_t rows,
                                                     int64_t ld, const int64_t* __restrict__ len,
                                                     int64_t ncols, int64_t lo, int64_t hi) {
  const int64_t total = rows * ncols;
  unsigned int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / ncols, c = i % ncols;
    int64_t n = ncols;
    if (len) {
      const int64_t l = len[r];
      n = l < 0 ? 0 : (l < ncols ? l : ncols);
    }
    if (c < n) {
      const int64_t v = a[r * ld + c];
      bad += (v < lo || v >= hi) ? 1u : 0u;
    }
  }
  if (bad) atomicAdd(&g_bad_count, bad);
}

hipError_t check_range(const int32_t* a, int64_t rows, int64_t ld, const int64_t* len,
                       int64_t ncols, int64_t lo, int64_t hi, hipStream_t stream,
                       unsigned int* bad) {
  *bad = 0;
  if (rows <= 0 || ncols <= 0) return hipSuccess;
  const unsigned int zero = 0;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_bad_count), &zero, sizeof(zero), 0,
                                        hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  const int64_t total = rows * ncols;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_check_range, dim3((unsigned)blocks), dim3(256), 0, stream, a, rows, ld, len,
                     ncols, lo, hi);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(bad, HIP_SYMBOL(g_bad_count), sizeof(*bad), 0,
                               hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

}  // namespace csa2
