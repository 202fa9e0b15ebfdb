// Projection-replay decode step, plain float32 FMA version: one workgroup per (request, beam, head).
//
// Serves every shape and the float32 inputs, and is the A/B partner of the fused bf16-MFMA kernel.
// Per pair, with the beam's chain (parent's history) j = 1..t-1 read from the ancestry index
// ("Scientific Impact Assessment: OneLA", §1 items (2)-(3); "Additional Observations"):
//   A   = prod_j alpha_j,   c_j = prod_{i after j} alpha_i
//   p   = A S_ctx k + sum_j c_j (K_j . k) U_j                 (= S_{t-1} k)
//   u   = beta (v - alpha p)                                   (the new record's vector)
//   o   = alpha (A S_ctx q + sum_j c_j (K_j . q) U_j) + (k . q) u   (= S_t q)
// and the record (alpha, k, u) is appended at slot (t-1) B_max + b.
#include "device_common.h"
#include "launchers.h"

namespace onela {

template <typename TIn>
__global__ __launch_bounds__(256) void step_generic_kernel(StepArgs a) {
  extern __shared__ float smem[];
  const int d_k = a.d_k, d_v = a.d_v, L = a.L_max;
  float* sk = smem;              // [d_k]
  float* sq = sk + d_k;          // [d_k]
  float* sdk = sq + d_k;         // [L] c_j (K_j . k)
  float* sdq = sdk + L;          // [L] c_j (K_j . q)
  float* sc = sdq + L;           // [L] c_j
  float* sal = sc + L;           // [L] alpha of chain records
  float* sA = sal + L;           // [1] A ; [2] k . q
  int* sslot = reinterpret_cast<int*>(sA + 4);  // [L]

  const int pair = blockIdx.x;
  const int h = pair % a.H;
  const int rb = pair / a.H;
  const int b = rb % a.n, r = rb / a.n;
  const int rh = r * a.H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = a.t - 1;
  const size_t in_row = ((size_t)r * a.n + b) * a.H + h;
  const TIn* kin = static_cast<const TIn*>(a.k) + in_row * d_k;
  const TIn* qin = static_cast<const TIn*>(a.q) + in_row * d_k;
  const TIn* vin = static_cast<const TIn*>(a.v) + in_row * d_v;
  const float alpha = a.alpha[in_row], beta = a.beta[in_row];
  const size_t arena = (size_t)rh * a.slots;
  const int own = (a.t - 1) * a.B_max + b;

  for (int i = tid; i < d_k; i += blockDim.x) {
    sk[i] = load_in(kin, i);
    sq[i] = load_in(qin, i);
  }
  const int32_t* ch = a.chain + ((size_t)r * a.B_max + b) * L;
  for (int m = tid; m < nch; m += blockDim.x) {
    int s = ch[m];
    s = s < 0 ? 0 : (s >= a.slots ? a.slots - 1 : s);
    sslot[m] = s;
    sal[m] = a.rec_alpha[arena + s];
  }
  __syncthreads();
  for (int m = tid; m < nch; m += blockDim.x) {
    float c = 1.f;
    for (int i = m + 1; i < nch; ++i) c *= sal[i];
    sc[m] = c;
  }
  if (tid == 0) {
    float A = 1.f;
    for (int i = 0; i < nch; ++i) A *= sal[i];
    sA[0] = A;
  }
  __syncthreads();
  // dot products with the chain keys (one wave per record) and k . q
  const TIn* rk = static_cast<const TIn*>(a.rec_k);
  for (int m = wave; m <= nch; m += blockDim.x >> 6) {
    float pk = 0.f, pq = 0.f;
    if (m < nch) {
      const TIn* K = rk + (arena + sslot[m]) * d_k;
      for (int d = lane; d < d_k; d += 64) {
        const float kv = load_in(K, d);
        pk += kv * sk[d];
        pq += kv * sq[d];
      }
    } else {
      for (int d = lane; d < d_k; d += 64) pk += sk[d] * sq[d];
    }
    pk = wave_sum(pk);
    pq = wave_sum(pq);
    if (lane == 0) {
      if (m < nch) {
        sdk[m] = sc[m] * pk;
        sdq[m] = sc[m] * pq;
      } else {
        sA[1] = pk;
      }
    }
  }
  __syncthreads();
  const float A = sA[0], kq = sA[1];
  const float* ST = a.sctx_t + (size_t)rh * d_k * d_v;
  for (int i = tid; i < d_v; i += blockDim.x) {
    float pk = 0.f, pq = 0.f;
    for (int d = 0; d < d_k; ++d) {
      const float s = ST[(size_t)d * d_v + i];
      pk += s * sk[d];
      pq += s * sq[d];
    }
    pk *= A;
    pq *= A;
    for (int m = 0; m < nch; ++m) {
      const float uu = a.rec_u[(arena + sslot[m]) * d_v + i];
      pk += sdk[m] * uu;
      pq += sdq[m] * uu;
    }
    const float u = beta * (load_in(vin, i) - alpha * pk);
    a.rec_u[(arena + own) * d_v + i] = u;
    a.o[in_row * d_v + i] = alpha * pq + kq * u;
  }
  TIn* rk_own = static_cast<TIn*>(a.rec_k) + (arena + own) * d_k;
  for (int i = tid; i < d_k; i += blockDim.x) rk_own[i] = kin[i];
  if (tid == 0) a.rec_alpha[arena + own] = alpha;
}

hipError_t launch_step_generic(const StepArgs& a, bool bf16, hipStream_t s) {
  const size_t lds = (size_t)(2 * a.d_k + 4 * a.L_max + 4) * sizeof(float) + (size_t)a.L_max * sizeof(int);
  dim3 grid((unsigned)((size_t)a.R * a.n * a.H)), block(256);
  if (bf16)
    hipLaunchKernelGGL(step_generic_kernel<uint16_t>, grid, block, lds, s, a);
  else
    hipLaunchKernelGGL(step_generic_kernel<float>, grid, block, lds, s, a);
  return hipGetLastError();
}

}  // namespace onela
