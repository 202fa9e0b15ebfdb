// Materializing-replay decode step: the comparison path that rebuilds each beam's dense state from the shared
// history every step ("Scientific Impact Assessment: OneLA", §1 and "Additional Observations": existing
// systems either keep a full state per beam or repeatedly replay the shared history; OneLA avoids both).
//
// One workgroup per (request, beam, head).  Thread (i, g) holds row i of the parent state in registers, for
// the d_k / G columns d = g, g + G, ...:
//   S_parent = A S_ctx + sum_j c_j U_j K_j^T          (the chain's records replayed onto S_ctx, densely)
//   p = S_parent k,  u = beta (v - alpha p),  o = alpha S_parent q + (k . q) u     (= S_t q)
// with A = prod alpha and c_j = prod of the alphas after record j along the chain.  It appends the same
// record (alpha, k, u) as the projection-replay kernels, so the two paths share the arenas, the ancestry
// index and the oracle.  The work is d_v d_k (t + 2) FMAs and a full read of S_ctx per pair and step,
// against d_v + d_k per record for projection replay.
#include "device_common.h"
#include "launchers.h"

namespace onela {

namespace {
constexpr int kMatCols = 64;  // columns of the state per thread (registers)
}

template <typename TIn, int G>
__global__ __launch_bounds__(1024) void step_materialize_kernel(StepArgs a) {
  extern __shared__ float smem[];
  const int d_k = a.d_k, d_v = a.d_v, L = a.L_max;
  float* sk = smem;              // [d_k]
  float* sq = sk + d_k;          // [d_k]
  float* sK = sq + d_k;          // [d_k] key of the record being replayed
  float* sU = sK + d_k;          // [d_v] its u
  float* sc = sU + d_v;          // [L] c_j
  float* sal = sc + L;           // [L] alpha of chain records
  float* red = sal + L;          // [2][G][d_v] partial projections
  float* sA = red + 2 * G * d_v; // [0] A, [1] k . q
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

  for (int x = tid; x < d_k; x += blockDim.x) {
    sk[x] = load_in(kin, x);
    sq[x] = load_in(qin, x);
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
    for (int x = m + 1; x < nch; ++x) c *= sal[x];
    sc[m] = c;
  }
  if (tid == 0) {
    float A = 1.f;
    for (int x = 0; x < nch; ++x) A *= sal[x];
    sA[0] = A;
  }
  if (wave == 0) {
    float kq = 0.f;
    for (int d = lane; d < d_k; d += 64) kq += sk[d] * sq[d];
    kq = wave_sum(kq);
    if (lane == 0) sA[1] = kq;
  }
  __syncthreads();

  // ---- S_parent = A S_ctx + sum_j c_j U_j K_j^T, row i of it in this thread's registers ----
  const bool owner = tid < d_v * G;
  const int i = tid % d_v, g = tid / d_v;
  const float A = sA[0];
  const int cpt = (d_k - g + G - 1) / G;  // this thread's columns: d = g + m G, m < cpt
  const float* ST = a.sctx_t + (size_t)rh * d_k * d_v;  // S_ctx transposed: [d_k][d_v]
  float S[kMatCols];
#pragma unroll
  for (int m = 0; m < kMatCols; ++m) {
    const int d = g + m * G;
    S[m] = owner && m < cpt ? A * ST[(size_t)d * d_v + i] : 0.f;
  }
  const TIn* rk = static_cast<const TIn*>(a.rec_k);
  for (int j = 0; j < nch; ++j) {
    for (int x = tid; x < d_k; x += blockDim.x) sK[x] = load_in(rk + (arena + sslot[j]) * d_k, x);
    for (int x = tid; x < d_v; x += blockDim.x) sU[x] = a.rec_u[(arena + sslot[j]) * d_v + x];
    __syncthreads();
    if (owner) {
      const float cu = sc[j] * sU[i];
#pragma unroll
      for (int m = 0; m < kMatCols; ++m) {
        if (m < cpt) S[m] += cu * sK[g + m * G];
      }
    }
    __syncthreads();
  }

  // ---- the two projections of the materialized state ----
  if (owner) {
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int m = 0; m < kMatCols; ++m) {
      if (m < cpt) {
        pk += S[m] * sk[g + m * G];
        pq += S[m] * sq[g + m * G];
      }
    }
    red[g * d_v + i] = pk;
    red[(G + g) * d_v + i] = pq;
  }
  __syncthreads();
  if (tid < d_v) {
    float pk = 0.f, pq = 0.f;
    for (int x = 0; x < G; ++x) {
      pk += red[x * d_v + tid];
      pq += red[(G + x) * d_v + tid];
    }
    const float u = beta * (load_in(vin, tid) - alpha * pk);
    a.rec_u[(arena + own) * d_v + tid] = u;
    a.o[in_row * d_v + tid] = alpha * pq + sA[1] * u;
  }
  TIn* rk_own = static_cast<TIn*>(a.rec_k) + (arena + own) * d_k;
  for (int x = tid; x < d_k; x += blockDim.x) rk_own[x] = kin[x];
  if (tid == 0) a.rec_alpha[arena + own] = alpha;
}

hipError_t launch_step_materialize(const StepArgs& a, bool bf16, hipStream_t s) {
  // G column groups of at most kMatCols columns each; d_v * G threads (at most 256 * 4 = 1024)
  const int G = (a.d_k + kMatCols - 1) / kMatCols;
  const int threads = ((a.d_v * G + 63) / 64) * 64;
  const size_t lds = (size_t)(3 * a.d_k + a.d_v + 2 * a.L_max + 2 * G * a.d_v + 4) * sizeof(float) +
                     (size_t)a.L_max * sizeof(int);
  dim3 grid((unsigned)((size_t)a.R * a.n * a.H)), block(threads);
#define ONELA_MAT_CASE(GG)                                                                       \
  case GG:                                                                                       \
    if (bf16)                                                                                    \
      hipLaunchKernelGGL((step_materialize_kernel<uint16_t, GG>), grid, block, lds, s, a);       \
    else                                                                                         \
      hipLaunchKernelGGL((step_materialize_kernel<float, GG>), grid, block, lds, s, a);          \
    break;
  switch (G) {
    ONELA_MAT_CASE(1)
    ONELA_MAT_CASE(2)
    ONELA_MAT_CASE(3)
    ONELA_MAT_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef ONELA_MAT_CASE
  return hipGetLastError();
}

}  // namespace onela
