// Materializing-replay decode step: the comparison path that rebuilds each beam's dense state from the shared
// history every step ("Scientific Impact Assessment: OneLA", §1 and "Additional Observations": existing
// systems either keep a full state per beam or repeatedly replay the shared history; OneLA avoids both).
//
// step_materialize_kernel: one workgroup per (request, beam, head) (the fallback for the widest shapes);
// step_materialize_tile_kernel below: one per 16 beams of a (request, head).  Thread (i, g) holds row i of the
// parent state in registers, for the columns d = g, g + G, ...:
//   S_parent = A S_ctx + sum_j c_j U_j K_j^T          (the chain's records replayed onto S_ctx, densely)
//   p = S_parent k,  u = beta (v - alpha p),  o = alpha S_parent q + (k . q) u     (= S_t q)
// with A = prod alpha and c_j = prod of the alphas after record j along the chain.  It appends the same
// record (alpha, k, u) as the projection-replay kernels, so the two paths share the arenas, the ancestry
// index and the oracle.  The work is d_v d_k (t + 2) FMAs per pair and step (and, in the per-pair kernel, a
// full read of S_ctx), against d_v + d_k per record for projection replay.
#include "device_common.h"
#include "launchers.h"

namespace onela {

namespace {
constexpr int kMatCols = 64;  // columns of the state per thread (registers)
constexpr int kMatRec = 8;    // chain records staged in LDS per pass (tile kernel)
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

// The same step for a tile of kMatTile beams of one (request, head) per workgroup: the S_ctx columns a thread
// owns are loaded into registers once and reused by every beam of the tile, so the dense rebuild is bound by
// its FMAs rather than by re-reading S_ctx for each beam.  Thread (i, g) holds row i for the kTileCols
// consecutive columns from g kTileCols (G = ceil(d_k / kTileCols)), so the key values it needs are 16-byte
// LDS broadcasts; each beam's chain records go through LDS kMatRec at a time.
constexpr int kMatTile = 16;
constexpr int kTileCols = 32;

template <typename TIn, int G>
__global__ __launch_bounds__(1024) void step_materialize_tile_kernel(StepArgs a, int ntile) {
  extern __shared__ __align__(16) float smem[];
  const int d_k = a.d_k, d_v = a.d_v, L = a.L_max;
  const int d_kp = G * kTileCols;          // key rows padded with zeros to the threads' column blocks
  float* sk = smem;                         // [kMatTile][d_kp]
  float* sq = sk + kMatTile * d_kp;         // [kMatTile][d_kp]
  float* sK = sq + kMatTile * d_kp;         // [kMatRec][d_kp]
  float* sU = sK + kMatRec * d_kp;          // [kMatRec][d_v]
  float* sc = sU + kMatRec * d_v;           // [kMatTile][L] c_j (alpha of record j until the products are formed)
  float* red = sc + kMatTile * L;           // [2][G][d_v]
  float* sA = red + 2 * G * d_v;            // [kMatTile] A
  float* skq = sA + kMatTile;               // [kMatTile] k . q
  float* sab = skq + kMatTile;              // [kMatTile][2] alpha, beta
  int* sslot = reinterpret_cast<int*>(sab + 2 * kMatTile);  // [kMatTile][L]

  const int tile = blockIdx.x % ntile, rh = blockIdx.x / ntile;
  const int h = rh % a.H, r = rh / a.H;
  const int b0 = tile * kMatTile, nbt = min(kMatTile, a.n - b0);
  const int tid = threadIdx.x, nthreads = blockDim.x;
  const int nch = a.t - 1;
  const size_t arena = (size_t)rh * a.slots;
  auto in_row = [&](int bb) { return ((size_t)r * a.n + b0 + bb) * a.H + h; };

  // the tile's k, q, alpha, beta; its chains and their records' alphas
  for (int x = tid; x < nbt * d_kp; x += nthreads) {
    const int bb = x / d_kp, d = x - bb * d_kp;
    sk[x] = d < d_k ? load_in(static_cast<const TIn*>(a.k) + in_row(bb) * d_k, d) : 0.f;
    sq[x] = d < d_k ? load_in(static_cast<const TIn*>(a.q) + in_row(bb) * d_k, d) : 0.f;
  }
  for (int bb = tid; bb < nbt; bb += nthreads) {
    sab[2 * bb] = a.alpha[in_row(bb)];
    sab[2 * bb + 1] = a.beta[in_row(bb)];
  }
  for (int x = tid; x < nbt * nch; x += nthreads) {
    const int bb = x / nch, m = x - bb * nch;
    int sl = a.chain[((size_t)r * a.B_max + b0 + bb) * L + m];
    sl = sl < 0 ? 0 : (sl >= a.slots ? a.slots - 1 : sl);
    sslot[bb * L + m] = sl;
    sc[bb * L + m] = a.rec_alpha[arena + sl];
  }
  // S_ctx columns of this thread, in registers for the whole tile
  const bool owner = tid < d_v * G;
  const int i = tid % d_v, g = tid / d_v;
  const int c0 = g * kTileCols, cpt = max(0, min(kTileCols, d_k - c0));  // columns c0 .. c0 + cpt - 1
  const float* ST = a.sctx_t + (size_t)rh * d_k * d_v;
  float Sc[kTileCols];
#pragma unroll
  for (int m = 0; m < kTileCols; ++m) Sc[m] = owner && m < cpt ? ST[(size_t)(c0 + m) * d_v + i] : 0.f;
  __syncthreads();
  for (int bb = tid; bb < nbt; bb += nthreads) {  // decay products along each chain, k . q
    float A = 1.f;
    for (int m = nch - 1; m >= 0; --m) {
      const float al = sc[bb * L + m];
      sc[bb * L + m] = A;  // product of the alphas after record m
      A *= al;
    }
    sA[bb] = A;
    float kq = 0.f;
    for (int d = 0; d < d_k; ++d) kq += sk[bb * d_kp + d] * sq[bb * d_kp + d];
    skq[bb] = kq;
  }
  __syncthreads();

  const TIn* rk = static_cast<const TIn*>(a.rec_k);
  for (int bb = 0; bb < nbt; ++bb) {
    float S[kTileCols];
    const float A = sA[bb];
#pragma unroll
    for (int m = 0; m < kTileCols; ++m) S[m] = A * Sc[m];
    for (int j0 = 0; j0 < nch; j0 += kMatRec) {  // the beam's records, kMatRec per pass
      const int nj = min(kMatRec, nch - j0);
      for (int x = tid; x < nj * d_kp; x += nthreads) {
        const int jj = x / d_kp, c = x - jj * d_kp;
        sK[x] = c < d_k ? load_in(rk + (arena + sslot[bb * L + j0 + jj]) * d_k, c) : 0.f;
      }
      for (int x = tid; x < nj * d_v; x += nthreads) {
        const int jj = x / d_v, c = x - jj * d_v;
        sU[x] = a.rec_u[(arena + sslot[bb * L + j0 + jj]) * d_v + c];
      }
      __syncthreads();
      if (owner) {
        for (int jj = 0; jj < nj; ++jj) {
          const float cu = sc[bb * L + j0 + jj] * sU[jj * d_v + i];
          const float* kj = sK + jj * d_kp + c0;  // every lane of a wave reads the same 16 bytes (broadcast)
#pragma unroll
          for (int m4 = 0; m4 < kTileCols; m4 += 4) {
            const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kj + m4);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m4 + e] += cu * kv[e];
          }
        }
      }
      __syncthreads();
    }
    // the two projections of the beam's materialized state
    if (owner) {
      float pk = 0.f, pq = 0.f;
      const float* kb = sk + bb * d_kp + c0;
      const float* qb = sq + bb * d_kp + c0;
#pragma unroll
      for (int m4 = 0; m4 < kTileCols; m4 += 4) {
        const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kb + m4);
        const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(qb + m4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk += S[m4 + e] * kv[e];
          pq += S[m4 + e] * qv[e];
        }
      }
      red[g * d_v + i] = pk;
      red[(G + g) * d_v + i] = pq;
    }
    __syncthreads();
    const size_t row = in_row(bb);
    const int own = nch * a.B_max + b0 + bb;
    if (tid < d_v) {
      float pk = 0.f, pq = 0.f;
      for (int x = 0; x < G; ++x) {
        pk += red[x * d_v + tid];
        pq += red[(G + x) * d_v + tid];
      }
      const float alpha = sab[2 * bb], beta = sab[2 * bb + 1];
      const float u = beta * (load_in(static_cast<const TIn*>(a.v) + row * d_v, tid) - alpha * pk);
      a.rec_u[(arena + own) * d_v + tid] = u;
      a.o[row * d_v + tid] = alpha * pq + skq[bb] * u;
    }
    TIn* rk_own = static_cast<TIn*>(a.rec_k) + (arena + own) * d_k;
    const TIn* kin = static_cast<const TIn*>(a.k) + row * d_k;
    for (int x = tid; x < d_k; x += nthreads) rk_own[x] = kin[x];
    if (tid == 0) a.rec_alpha[arena + own] = sab[2 * bb];
    __syncthreads();  // red is rewritten by the next beam
  }
}

hipError_t launch_step_materialize(const StepArgs& a, bool bf16, hipStream_t s) {
  {  // tiles of beams sharing the S_ctx columns in registers, when d_v * G threads fit one workgroup
    const int G = (a.d_k + kTileCols - 1) / kTileCols;
    if (G <= 8 && a.d_v * G <= 1024) {
      const int threads = ((a.d_v * G + 63) / 64) * 64;
      const int ntile = (a.n + kMatTile - 1) / kMatTile;
      const int d_kp = G * kTileCols;
      const size_t lds = (size_t)(2 * kMatTile * d_kp + kMatRec * (d_kp + a.d_v) + kMatTile * a.L_max +
                                  2 * G * a.d_v + 4 * kMatTile) * sizeof(float) +
                         (size_t)kMatTile * a.L_max * sizeof(int);
      dim3 grid((unsigned)((size_t)a.R * a.H * ntile)), block(threads);
#define ONELA_MATT_CASE(GG)                                                                                    \
  case GG:                                                                                                     \
    if (lds > 64 * 1024) {                                                                                     \
      hipError_t e = hipFuncSetAttribute(                                                                      \
          bf16 ? reinterpret_cast<const void*>(&step_materialize_tile_kernel<uint16_t, GG>)                    \
               : reinterpret_cast<const void*>(&step_materialize_tile_kernel<float, GG>),                      \
          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                                               \
      if (e != hipSuccess) return e;                                                                           \
    }                                                                                                          \
    if (bf16)                                                                                                  \
      hipLaunchKernelGGL((step_materialize_tile_kernel<uint16_t, GG>), grid, block, lds, s, a, ntile);         \
    else                                                                                                       \
      hipLaunchKernelGGL((step_materialize_tile_kernel<float, GG>), grid, block, lds, s, a, ntile);            \
    break;
      switch (G) {
        ONELA_MATT_CASE(1)
        ONELA_MATT_CASE(2)
        ONELA_MATT_CASE(3)
        ONELA_MATT_CASE(4)
        ONELA_MATT_CASE(5)
        ONELA_MATT_CASE(6)
        ONELA_MATT_CASE(7)
        ONELA_MATT_CASE(8)
        default:
          return hipErrorInvalidValue;
      }
#undef ONELA_MATT_CASE
      return hipGetLastError();
    }
  }
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
