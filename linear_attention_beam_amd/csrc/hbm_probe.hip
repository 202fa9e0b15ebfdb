// Streaming probes of the HBM bandwidth a plain kernel reaches on this GPU, for the bench's context figures
// (the roofline peak itself stays the published 8 TB/s).  Separate library (libonela_probe.so): measurement
// infrastructure, not part of the decode path.  Every access is a 16-byte load or store, consecutive lanes on
// consecutive addresses, in n-element streams:
//   mode 0 read    sums src[0 .. 2n) (in the grid-stride form one float per thread is written at the end)
//   mode 1 mix     reads src[i], src[n + i]; writes dst[i], dst[n + i], dst[2n + i]: 2 bytes read for every
//                  3 written, the mix of the decode step (q, k, v, S_ctx and records in; o, u, k records out)
//   mode 2 copy    dst[i] = src[i], i < n
//   mode 3 write   dst[i] = constant, i < n
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "onela_probe.h"

namespace {
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One element per thread (grid covers n) when stride == 0, else a grid-stride loop.
__global__ __launch_bounds__(256) void probe_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, size_t n,
                                                    int mode, float* __restrict__ sink, int strided) {
  const size_t stride = strided ? (size_t)gridDim.x * blockDim.x : 2 * n + 1;
  const size_t first = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (mode == 0) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (size_t i = first; i < n; i += stride) acc += src[i] + src[n + i];
    const float v = acc.x + acc.y + acc.z + acc.w;
    if (strided || v == -1.2345f) sink[strided ? first : 0] = v;  // one-element form: kept live, almost never written
  } else if (mode == 1) {
    for (size_t i = first; i < n; i += stride) {
      const f32x4 a = src[i], b = src[n + i];
      dst[i] = a;
      dst[n + i] = b;
      dst[2 * n + i] = a + b;
    }
  } else if (mode == 2) {
    for (size_t i = first; i < n; i += stride) dst[i] = src[i];
  } else {
    const f32x4 c = {1.f, 2.f, 3.f, 4.f};
    for (size_t i = first; i < n; i += stride) dst[i] = c;
  }
}
}  // namespace

extern "C" int onela_probe_stream(const void* src, void* dst, size_t n, int mode, float* sink, int grid,
                                  void* stream) {
  if (mode < 0 || mode > 3 || grid < 0 || n == 0) return 1;
  if ((mode != 3 && !src) || (mode != 0 && !dst) || (mode == 0 && !sink)) return 1;
  const size_t blocks = grid ? (size_t)grid : (n + 255) / 256;
  if (blocks > 0x7FFFFFFFu) return 1;
  hipLaunchKernelGGL(probe_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n, mode, sink, grid ? 1 : 0);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
