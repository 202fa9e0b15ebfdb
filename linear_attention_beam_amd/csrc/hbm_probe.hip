// Streaming probes of the HBM bandwidth a plain kernel reaches on this GPU, for the bench's context figures
// (the roofline peak itself stays the published 8 TB/s).  Separate library (libonela_probe.so): measurement
// infrastructure, not part of the decode path.  Every access is a 16-byte load or store, consecutive lanes on
// consecutive addresses, in n-element streams:
//   mode 0 read    sums src[0 .. 2n) (in the grid-stride form one float per thread is written at the end)
//   mode 1 mix     reads src[i], src[n + i]; writes dst[i], dst[n + i], dst[2n + i]: 2 bytes read for every
//                  3 written, the mix of the decode step (q, k, v, S_ctx and records in; o, u, k records out)
//   mode 2 copy    dst[i] = src[i], i < n
//   mode 3 write   dst[i] = constant, i < n
// and the first decode step's traffic without its arithmetic (onela_probe_step_traffic): the same rows read and
// written, from plain workgroups with no LDS and no barriers.
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (request, head, tile of 32 beams), blockIdx = (request * H + head) * (B / 32) + tile.  Each
// thread issues all its loads at once (its pieces of the tile's k, q and v rows, of alpha and beta, and of the
// tile's share of the head's S_ctx), then stores its pieces of the o, u and key rows and of alpha, with values
// folded from what it loaded so that no load is dead.
template <int DV>
__global__ __launch_bounds__(256) void step_traffic_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ q,
    const u32x4* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    const u32x4* __restrict__ sctx, u32x4* __restrict__ o, u32x4* __restrict__ u, u32x4* __restrict__ rec_k,
    float* __restrict__ rec_alpha, int B, int H, int slots) {
  constexpr int VP = DV / 8, OP = DV / 4;            // 16-byte pieces of a v row (bf16), of an o or u row (fp32)
  constexpr int NV = (32 * VP + 255) / 256, NO = 32 * OP / 256;
  const int ntile = B / 32, tid = threadIdx.x;
  const int rh = blockIdx.x / ntile, tile = blockIdx.x - rh * ntile, r = rh / H, h = rh - r * H;
  const size_t row0 = ((size_t)r * B + tile * 32) * H + h;  // input row of the tile's first beam
  u32x4 kk[2], qq[2], vv[NV];
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // k and q: 32 rows of 16 pieces
    const int p = i * 256 + tid;
    kk[i] = k[(row0 + (size_t)(p >> 4) * H) * 16 + (p & 15)];
    qq[i] = q[(row0 + (size_t)(p >> 4) * H) * 16 + (p & 15)];
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int p = min(i * 256 + tid, 32 * VP - 1);
    vv[i] = v[(row0 + (size_t)(p / VP) * H) * VP + p % VP];
  }
  const size_t ab_i = row0 + (size_t)(tid & 31) * H;
  const float ab = alpha[ab_i] + beta[ab_i];
  // this tile's share of the head's S_ctx (128 x DV float32 = 32 * DV pieces)
  const int per = (32 * DV + ntile - 1) / ntile, s0 = tile * per, s1 = min(32 * DV, s0 + per);
  u32x4 acc = kk[0] ^ kk[1] ^ qq[0] ^ qq[1];
#pragma unroll 4
  for (int p = s0 + tid; p < s1; p += 256) acc ^= sctx[(size_t)rh * 32 * DV + p];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc ^= vv[i];
#pragma unroll
  for (int i = 0; i < NO; ++i) {
    const int p = i * 256 + tid;
    const u32x4 x = acc ^ (u32x4){(unsigned)p, 0u, 0u, 0u};
    o[(row0 + (size_t)(p / OP) * H) * OP + p % OP] = x & 0x3fffffffu;
    u[((size_t)rh * slots + tile * 32 + p / OP) * OP + p % OP] = x & 0x3effffffu;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = i * 256 + tid;
    rec_k[((size_t)rh * slots + tile * 32 + (p >> 4)) * 16 + (p & 15)] = kk[i];
  }
  if (tid < 32) rec_alpha[(size_t)rh * slots + tile * 32 + tid] = ab;
}
using StepTrafficKernel = void (*)(const u32x4*, const u32x4*, const u32x4*, const float*, const float*,
                                   const u32x4*, u32x4*, u32x4*, u32x4*, float*, int, int, int);
StepTrafficKernel step_traffic_for(int d_v) {
  switch (d_v) {
    case 32: return &step_traffic_kernel<32>;
    case 64: return &step_traffic_kernel<64>;
    case 96: return &step_traffic_kernel<96>;
    case 128: return &step_traffic_kernel<128>;
    case 160: return &step_traffic_kernel<160>;
    case 192: return &step_traffic_kernel<192>;
    case 224: return &step_traffic_kernel<224>;
    case 256: return &step_traffic_kernel<256>;
    default: return nullptr;
  }
}
}  // namespace

extern "C" int onela_probe_step_traffic(const void* k, const void* q, const void* v, const float* alpha,
                                        const float* beta, const void* sctx, void* o, void* u, void* rec_k,
                                        float* rec_alpha, int R, int B, int H, int d_v, int slots, void* stream) {
  if (!k || !q || !v || !alpha || !beta || !sctx || !o || !u || !rec_k || !rec_alpha) return 1;
  if (R <= 0 || H <= 0 || B <= 0 || B % 32 || d_v <= 0 || d_v % 32 || d_v > 256 || slots < B) return 1;
  const long blocks = (long)R * H * (B / 32);
  if (blocks > 0x7FFFFFFFL) return 1;
  hipLaunchKernelGGL(step_traffic_for(d_v), dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(q), static_cast<const u32x4*>(v), alpha,
                     beta, static_cast<const u32x4*>(sctx), static_cast<u32x4*>(o), static_cast<u32x4*>(u),
                     static_cast<u32x4*>(rec_k), rec_alpha, B, H, slots);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

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
