// FullState decode step: the controlled comparison ("Scientific Impact Assessment: OneLA", §2: the
// Controlled FullState baseline keeps the decode pipeline and swaps in a dense state per beam; paper
// index page, Abstract: systems that materialise a full recurrent state for every beam).
//
// One workgroup of 256 threads per (request, beam, head).  The parent's state S_p (stored transposed,
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

hipError_t launch_fullstate(const StepArgs& a, bool bf16, const int32_t* parent, int b_prev, const float* fs_prev,
                            float* fs_next, hipStream_t s) {
  const size_t lds = (size_t)(2 * a.d_k + 512 + a.d_v + 4) * sizeof(float);
  dim3 grid((unsigned)((size_t)a.R * a.n * a.H)), block(256);
  if (bf16)
    hipLaunchKernelGGL(fullstate_kernel<uint16_t>, grid, block, lds, s, a, parent, b_prev, fs_prev, fs_next);
  else
    hipLaunchKernelGGL(fullstate_kernel<float>, grid, block, lds, s, a, parent, b_prev, fs_prev, fs_next);
  return hipGetLastError();
}

}  // namespace onela
