// FullState decode step: the controlled comparison ("Scientific Impact Assessment: OneLA", §2: the
// Controlled FullState baseline keeps the decode pipeline and swaps in a dense state per beam; paper
// index page, Abstract: systems that materialise a full recurrent state for every beam).
//
// One workgroup of 256 threads per (request, beam, head) (the kernel for d_v % 4 != 0).  The parent's state S_p (stored transposed,
// [d_k][d_v], so that threads walking d_v read contiguous memory; S_ctx^T at step 1) is read once to form
// S_p k and S_p q, then read again to write the child's state:
//   u = beta (v - alpha S_p k),  S = alpha S_p + u k^T,  o = S q = alpha S_p q + (k . q) u.
// Thread (i, part) owns column i of S^T for the keys of its part (NPART = 256 / d_v parts, d_v <= 256).
#include "device_common.h"
#include "launchers.h"

namespace onela {

template <typename TIn>
__global__ __launch_bounds__(256) void fullstate_kernel(StepArgs a, const int32_t* __restrict__ parent, int b_prev,
                                                        const float* __restrict__ fs_prev, float* __restrict__ fs_next) {
  extern __shared__ float smem[];
  const int d_k = a.d_k, d_v = a.d_v;
  float* sk = smem;            // [d_k]
  float* sq = sk + d_k;        // [d_k]
  float* part_k = sq + d_k;    // [256]
  float* part_q = part_k + 256;
  float* su = part_q + 256;    // [d_v]
  float* skq = su + d_v;       // [1]

  const int pair = blockIdx.x;
  const int h = pair % a.H;
  const int rb = pair / a.H;
  const int b = rb % a.n, r = rb / a.n;
  const int rh = r * a.H + h;
  const int tid = threadIdx.x;
  const size_t in_row = ((size_t)r * a.n + b) * a.H + h;
  const TIn* kin = static_cast<const TIn*>(a.k) + in_row * d_k;
  const TIn* qin = static_cast<const TIn*>(a.q) + in_row * d_k;
  const TIn* vin = static_cast<const TIn*>(a.v) + in_row * d_v;
  const float alpha = a.alpha[in_row], beta = a.beta[in_row];
  int p = parent[(size_t)r * a.n + b];
  if (p < 0 || p >= b_prev) p = 0;  // flagged by the ancestry kernel
  const size_t state = (size_t)d_k * d_v;
  const float* Sp = a.t == 1 ? a.sctx_t + (size_t)rh * state
                             : fs_prev + (((size_t)r * a.H + h) * a.B_max + p) * state;
  float* Sn = fs_next + (((size_t)r * a.H + h) * a.B_max + b) * state;

  for (int i = tid; i < d_k; i += 256) {
    sk[i] = load_in(kin, i);
    sq[i] = load_in(qin, i);
  }
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
    for (int d = tid; d < d_k; d += 64) s += sk[d] * sq[d];
    s = wave_sum(s);
    if (tid == 0) skq[0] = s;
  }
  const int nparts = 256 / d_v;
  const int i = tid % d_v, part = tid / d_v;
  const int per = (d_k + nparts - 1) / nparts;
  const int d0 = part * per, d1 = min(d_k, d0 + per);
  float pk = 0.f, pq = 0.f;
  for (int d = d0; d < d1; ++d) {
    const float s = Sp[(size_t)d * d_v + i];
    pk += s * sk[d];
    pq += s * sq[d];
  }
  part_k[tid] = pk;
  part_q[tid] = pq;
  __syncthreads();
  if (part == 0) {
    float tk = 0.f, tq = 0.f;
    for (int q = 0; q < nparts; ++q) {
      tk += part_k[q * d_v + i];
      tq += part_q[q * d_v + i];
    }
    const float u = beta * (load_in(vin, i) - alpha * tk);
    su[i] = u;
    a.o[in_row * d_v + i] = alpha * tq + skq[0] * u;
  }
  __syncthreads();
  const float u = su[i];
  for (int d = d0; d < d1; ++d) Sn[(size_t)d * d_v + i] = alpha * Sp[(size_t)d * d_v + i] + u * sk[d];
}

// Same step, state read once: thread (c, g) holds columns 4c .. 4c+3 of S_p^T for the 16 keys 16g .. 16g+15 in
// registers (d_v % 4 == 0), loads and stores them as 16-byte pieces, and the partial projections of the G =
// ceil(d_k / 16) key groups are summed through LDS.
template <typename TIn>
__global__ __launch_bounds__(1024) void fullstate4_kernel(StepArgs a, const int32_t* __restrict__ parent, int b_prev,
                                                          const float* __restrict__ fs_prev,
                                                          float* __restrict__ fs_next) {
  extern __shared__ float smem[];
  constexpr int kKeys = 16;
  const int d_k = a.d_k, d_v = a.d_v, nc = d_v >> 2, G = (d_k + kKeys - 1) / kKeys;
  float* sk = smem;                 // [G * 16] (zero past d_k)
  float* sq = sk + G * kKeys;
  float* part = sq + G * kKeys;     // [2][G][d_v]
  float* skq = part + 2 * G * d_v;  // [1]

  const int pair = blockIdx.x;
  const int h = pair % a.H;
  const int rb = pair / a.H;
  const int b = rb % a.n, r = rb / a.n;
  const int rh = r * a.H + h;
  const int tid = threadIdx.x;
  const size_t in_row = ((size_t)r * a.n + b) * a.H + h;
  const TIn* kin = static_cast<const TIn*>(a.k) + in_row * d_k;
  const TIn* qin = static_cast<const TIn*>(a.q) + in_row * d_k;
  const TIn* vin = static_cast<const TIn*>(a.v) + in_row * d_v;
  const float alpha = a.alpha[in_row], beta = a.beta[in_row];
  int p = parent[(size_t)r * a.n + b];
  if (p < 0 || p >= b_prev) p = 0;  // flagged by the ancestry kernel
  const size_t state = (size_t)d_k * d_v;
  const float* Sp = a.t == 1 ? a.sctx_t + (size_t)rh * state
                             : fs_prev + (((size_t)r * a.H + h) * a.B_max + p) * state;
  float* Sn = fs_next + (((size_t)r * a.H + h) * a.B_max + b) * state;

  const bool owner = tid < nc * G;
  const int c = tid % nc, g = tid / nc;
  const int d0 = g * kKeys, cnt = owner ? max(0, min(kKeys, d_k - d0)) : 0;
  f32x4_t S[kKeys];
#pragma unroll
  for (int e = 0; e < kKeys; ++e)
    S[e] = e < cnt ? *reinterpret_cast<const f32x4_t*>(Sp + (size_t)(d0 + e) * d_v + 4 * c)
                   : (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int x = tid; x < G * kKeys; x += blockDim.x) {
    sk[x] = x < d_k ? load_in(kin, x) : 0.f;
    sq[x] = x < d_k ? load_in(qin, x) : 0.f;
  }
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
    for (int d = tid; d < d_k; d += 64) s += sk[d] * sq[d];
    s = wave_sum(s);
    if (tid == 0) skq[0] = s;
  }
  f32x4_t pk = (f32x4_t){0.f, 0.f, 0.f, 0.f}, pq = pk;
  if (owner) {
#pragma unroll
    for (int e = 0; e < kKeys; ++e) {
      const float kk = sk[d0 + e], qq = sq[d0 + e];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pk[x] += S[e][x] * kk;
        pq[x] += S[e][x] * qq;
      }
    }
    *reinterpret_cast<f32x4_t*>(part + g * d_v + 4 * c) = pk;
    *reinterpret_cast<f32x4_t*>(part + (G + g) * d_v + 4 * c) = pq;
  }
  __syncthreads();
  if (!owner) return;
  f32x4_t tk = (f32x4_t){0.f, 0.f, 0.f, 0.f}, tq = tk;
  for (int x = 0; x < G; ++x) {
    tk += *reinterpret_cast<const f32x4_t*>(part + x * d_v + 4 * c);
    tq += *reinterpret_cast<const f32x4_t*>(part + (G + x) * d_v + 4 * c);
  }
  f32x4_t u, o;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    u[x] = beta * (load_in(vin, 4 * c + x) - alpha * tk[x]);
    o[x] = alpha * tq[x] + skq[0] * u[x];
  }
  if (g == 0) *reinterpret_cast<f32x4_t*>(a.o + in_row * d_v + 4 * c) = o;
#pragma unroll
  for (int e = 0; e < kKeys; ++e) {
    if (e < cnt) {
      const float kk = sk[d0 + e];
      f32x4_t n;
#pragma unroll
      for (int x = 0; x < 4; ++x) n[x] = alpha * S[e][x] + u[x] * kk;
      *reinterpret_cast<f32x4_t*>(Sn + (size_t)(d0 + e) * d_v + 4 * c) = n;
    }
  }
}

hipError_t launch_fullstate(const StepArgs& a, bool bf16, const int32_t* parent, int b_prev, const float* fs_prev,
                            float* fs_next, hipStream_t s) {
  dim3 grid((unsigned)((size_t)a.R * a.n * a.H));
  if (a.d_v % 4 == 0) {  // the state read once, in 16-byte pieces
    const int G = (a.d_k + 15) / 16;
    const int threads = ((a.d_v / 4 * G + 63) / 64) * 64;  // d_v / 4 * G <= 64 * 16
    const size_t lds4 = (size_t)(2 * G * 16 + 2 * G * a.d_v + 4) * sizeof(float);
    if (bf16)
      hipLaunchKernelGGL(fullstate4_kernel<uint16_t>, grid, dim3(threads), lds4, s, a, parent, b_prev, fs_prev,
                         fs_next);
    else
      hipLaunchKernelGGL(fullstate4_kernel<float>, grid, dim3(threads), lds4, s, a, parent, b_prev, fs_prev, fs_next);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(2 * a.d_k + 512 + a.d_v + 4) * sizeof(float);
  dim3 block(256);
  if (bf16)
    hipLaunchKernelGGL(fullstate_kernel<uint16_t>, grid, block, lds, s, a, parent, b_prev, fs_prev, fs_next);
  else
    hipLaunchKernelGGL(fullstate_kernel<float>, grid, block, lds, s, a, parent, b_prev, fs_prev, fs_next);
  return hipGetLastError();
}

}  // namespace onela
