// Fused projection-replay decode step for gfx950: bf16 MFMA contraction of the shared state, record
// replay and record append in one kernel ("Scientific Impact Assessment: OneLA", §1: a fused GPU kernel
// reuses S_ctx across beams; paper index page, Abstract).
//
// Workgroup = (request, head, tile of NB beams); d_v / 32 waves of 64 lanes (d_k = 128 fixed).
//   Phase 0  ancestry index ("Scientific Impact Assessment: OneLA", §1 item (3)): each beam's chain is
//            its parent's chain from the previous table plus its own slot; the head-0 workgroups write
//            the new table.  Stage k and q of the tile in LDS; read the chain records' alphas and form
//            the decays A = prod alpha and c_j = prod of the alphas after record j.
//   Phase 1  (16 lanes per beam) dot products of the chain keys with k and q, and k . q, reduced with
//            DPP inside a 16-lane row; append the record key and alpha.
//   Phase 2  each wave owns 32 columns of d_v.  For 16 beams at a time it runs
//            v_mfma_f32_16x16x32_bf16 over d_k: [P_k | P_q] = X^T S_ctx^T with X = [k | q], in two
//            passes over the bf16 high and low halves of S_ctx (the halves stay in registers for the
//            whole tile: each S_ctx element is read once per tile and reused by all NB beams).  The
//            accumulator layout (lane l: beam 4(l/16)+i, column l%16) is used as is: with the columns of
//            S_ctx^T permuted at split time, lane l holds d_v elements 32 w + 2 (l%16) + {0, 1}, so the
//            replay reads each record's u as contiguous float2 and writes u and o the same way:
//              p = A P_k + sum_j c_j (K_j.k) U_j,  u = beta (v - alpha p),
//              o = alpha (A P_q + sum_j c_j (K_j.q) U_j) + (k.q) u.
// Workgroups of one (request, head) are mapped to the same XCD (dispatch is round-robin over the 8 XCDs)
// so their S_ctx reads share one L2.
#include "device_common.h"
#include "launchers.h"

namespace onela {

namespace {
constexpr int kDK = 128;          // d_k of the fused kernel
constexpr int kKS = kDK / 32;     // MFMA k-steps
constexpr int kXRow = 2 * kDK + 16;  // bytes per staged key/query row (padded against bank conflicts)

struct FusedLds {
  int xs, slot, alph, coefk, coefq, beamA, beamAl, beamBe, beamKq, beamPar, total;
};

__host__ __device__ inline FusedLds fused_layout(int NB, int L) {
  FusedLds l;
  int off = 0;
  l.xs = off;     off += 2 * NB * kXRow;
  l.slot = off;   off += NB * L * 4;
  l.alph = off;   off += NB * L * 4;   // chain alphas, then c_j
  l.coefk = off;  off += NB * L * 4;
  l.coefq = off;  off += NB * L * 4;
  l.beamA = off;  off += NB * 4;
  l.beamAl = off; off += NB * 4;
  l.beamBe = off; off += NB * 4;
  l.beamKq = off; off += NB * 4;
  l.beamPar = off; off += NB * 4;
  l.total = off;
  return l;
}
}  // namespace

template <int NB>
__global__ __launch_bounds__(512) void step_fused_kernel(StepArgs a, int ntile) {
  extern __shared__ __align__(16) unsigned char lds[];
  const FusedLds lay = fused_layout(NB, a.L_max);
  unsigned char* xs = lds + lay.xs;
  int* slot_tab = reinterpret_cast<int*>(lds + lay.slot);
  float* c_tab = reinterpret_cast<float*>(lds + lay.alph);
  float* coefk = reinterpret_cast<float*>(lds + lay.coefk);
  float* coefq = reinterpret_cast<float*>(lds + lay.coefq);
  float* beamA = reinterpret_cast<float*>(lds + lay.beamA);
  float* beamAl = reinterpret_cast<float*>(lds + lay.beamAl);
  float* beamBe = reinterpret_cast<float*>(lds + lay.beamBe);
  float* beamKq = reinterpret_cast<float*>(lds + lay.beamKq);
  int* beamPar = reinterpret_cast<int*>(lds + lay.beamPar);

  const int L = a.L_max, H = a.H, n = a.n, d_v = a.d_v;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;

  // ---- workgroup -> (request, head, tile); tiles of one (request, head) share an XCD ----
  const int G = a.R * H;
  int rh, tile;
  if ((G & 7) == 0) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    rh = (j / ntile) * 8 + x;
    tile = j - (j / ntile) * ntile;
  } else {
    rh = blockIdx.x / ntile;
    tile = blockIdx.x - rh * ntile;
  }
  const int r = rh / H, h = rh - r * H;
  const int b0 = tile * NB;
  const int nb = min(NB, n - b0);
  const int nch = a.t - 1;
  const size_t arena = (size_t)rh * a.slots;
  const uint16_t* qin = static_cast<const uint16_t*>(a.q);
  const uint16_t* kin = static_cast<const uint16_t*>(a.k);
  const uint16_t* vin = static_cast<const uint16_t*>(a.v);
  uint16_t* rec_k = static_cast<uint16_t*>(a.rec_k);
  auto in_row = [&](int bb) { return ((size_t)r * n + b0 + bb) * H + h; };

  // ---- this wave's 32 columns of S_ctx^T, bf16 high and low halves, resident for the whole tile ----
  // fragment file per (request, head): [hl][w][ks][n][lane][8]
  bf16x8_t sf[kKS][2][2];
  {
    const int W = d_v / 32;
    const size_t half = (size_t)W * kKS * 2 * 64;  // fragments per half
    const u32x4_t* fr = reinterpret_cast<const u32x4_t*>(a.sctx_frag) + (size_t)rh * 2 * half;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int nn = 0; nn < 2; ++nn)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
          sf[ks][nn][hl] = __builtin_bit_cast(
              bf16x8_t, fr[hl * half + (((size_t)wave * kKS + ks) * 2 + nn) * 64 + lane]);
  }

  // ---- phase 0: parents, stage k and q, chains, chain alphas; per-beam alpha and beta ----
  for (int bb = tid; bb < NB; bb += nthreads) {
    const bool live = bb < nb;
    int p = 0;
    if (live) {
      p = a.parent[(size_t)r * n + b0 + bb];
      if (p < 0 || p >= a.b_prev) {  // sticky flag; decode as a child of beam 0 so accesses stay in bounds
        *a.flag = a.epoch;
        p = 0;
      }
    }
    beamPar[bb] = p;
    beamAl[bb] = live ? a.alpha[in_row(bb)] : 0.f;
    beamBe[bb] = live ? a.beta[in_row(bb)] : 0.f;
  }
  for (int idx = tid; idx < NB * 32; idx += nthreads) {
    const int row = idx >> 4, c = idx & 15;  // row < NB: key rows, row >= NB: query rows
    const int bb = row < NB ? row : row - NB;
    u32x4_t val = {0u, 0u, 0u, 0u};
    if (bb < nb) {
      const uint16_t* src = (row < NB ? kin : qin) + in_row(bb) * kDK + c * 8;
      val = *reinterpret_cast<const u32x4_t*>(src);
    }
    *reinterpret_cast<u32x4_t*>(xs + row * kXRow + c * 16) = val;
  }
  __syncthreads();
  for (int idx = tid; idx < nb * nch; idx += nthreads) {
    const int bb = idx / nch, m = idx - bb * nch;
    const int raw = a.chain_prev[((size_t)r * a.B_max + beamPar[bb]) * L + m];
    const int s = raw < 0 ? 0 : (raw >= a.slots ? a.slots - 1 : raw);
    slot_tab[bb * L + m] = s;
    c_tab[bb * L + m] = a.rec_alpha[arena + s];
    if (h == 0) a.chain_out[((size_t)r * a.B_max + b0 + bb) * L + m] = raw;
  }
  if (h == 0) {  // the rest of each row: own slot, then -1; rows of beams >= n are all -1
    for (int idx = tid; idx < nb * (L - nch); idx += nthreads) {
      const int bb = idx / (L - nch), m = nch + idx - bb * (L - nch);
      a.chain_out[((size_t)r * a.B_max + b0 + bb) * L + m] = m == nch ? nch * a.B_max + b0 + bb : -1;
    }
    if (tile == ntile - 1) {
      for (int idx = tid; idx < (a.B_max - n) * L; idx += nthreads)
        a.chain_out[((size_t)r * a.B_max + n) * L + idx] = -1;
    }
  }
  __syncthreads();
  for (int bb = tid; bb < NB; bb += nthreads) {  // alphas -> suffix products c_j, and A
    float run = 1.f;
    if (bb < nb) {
      for (int m = nch - 1; m >= 0; --m) {
        const float al = c_tab[bb * L + m];
        c_tab[bb * L + m] = run;
        run *= al;
      }
    }
    beamA[bb] = bb < nb ? run : 0.f;
  }
  __syncthreads();

  // ---- phase 1: chain-key dot products, 16 lanes per beam; append key and alpha ----
  {
    const int g = tid >> 4, j = tid & 15;
    const int ngroups = nthreads >> 4;
    for (int bb = g; bb < nb; bb += ngroups) {
      const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(xs + bb * kXRow + j * 16);
      const u32x4_t qx = *reinterpret_cast<const u32x4_t*>(xs + (NB + bb) * kXRow + j * 16);
      const int own = (a.t - 1) * a.B_max + b0 + bb;
      *reinterpret_cast<u32x4_t*>(rec_k + (arena + own) * kDK + j * 8) = kx;
      const float kq = row16_sum(dot8_bf16(kx, qx));
      for (int m0 = 0; m0 < nch; m0 += 4) {
        u32x4_t K[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int m = m0 + u < nch ? m0 + u : nch - 1;
          K[u] = *reinterpret_cast<const u32x4_t*>(rec_k + (arena + slot_tab[bb * L + m]) * kDK + j * 8);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float dk = row16_sum(dot8_bf16(K[u], kx));
          const float dq = row16_sum(dot8_bf16(K[u], qx));
          if (j == 0 && m0 + u < nch) {
            const float c = c_tab[bb * L + m0 + u];
            coefk[bb * L + m0 + u] = c * dk;
            coefq[bb * L + m0 + u] = c * dq;
          }
        }
      }
      if (j == 0) {
        beamKq[bb] = kq;
        a.rec_alpha[arena + own] = beamAl[bb];
      }
    }
  }
  __syncthreads();

  // ---- phase 2: MFMA contraction + replay + append, 16 beams per iteration ----
  const int gq = lane >> 4, col = lane & 15;
  const int dvi = wave * 32 + 2 * col;  // this lane's two d_v elements
  for (int mt = 0; mt * 16 < nb; ++mt) {
    floatx4_t pk[2], pq[2];
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      pk[nn] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
      pq[nn] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
    }
    const int arow = mt * 16 + col;  // A operand: lane l holds row l%16, k = 8 (l/16) .. +7
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const bf16x8_t ak =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + arow * kXRow + ks * 64 + gq * 16));
      const bf16x8_t aq = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + (NB + arow) * kXRow + ks * 64 + gq * 16));
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          pk[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, sf[ks][nn][hl], pk[nn], 0, 0, 0);
          pq[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, sf[ks][nn][hl], pq[nn], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bb = mt * 16 + 4 * gq + i;
      if (bb >= nb) continue;
      const float A = beamA[bb];
      float p0 = A * pk[0][i], p1 = A * pk[1][i];
      float s0 = A * pq[0][i], s1 = A * pq[1][i];
      for (int m0 = 0; m0 < nch; m0 += 4) {
        f32x2_t U[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int m = m0 + u < nch ? m0 + u : nch - 1;
          U[u] = *reinterpret_cast<const f32x2_t*>(a.rec_u + (arena + slot_tab[bb * L + m]) * d_v + dvi);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (m0 + u < nch) {
            const float ck = coefk[bb * L + m0 + u], cq = coefq[bb * L + m0 + u];
            p0 += ck * U[u].x;
            p1 += ck * U[u].y;
            s0 += cq * U[u].x;
            s1 += cq * U[u].y;
          }
        }
      }
      const size_t row = in_row(bb);
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(vin + row * d_v + dvi);
      const float al = beamAl[bb], be = beamBe[bb], kq = beamKq[bb];
      f32x2_t u2, o2;
      u2.x = be * (bf16_bits_to_f32(vv & 0xFFFFu) - al * p0);
      u2.y = be * (bf16_bits_to_f32(vv >> 16) - al * p1);
      o2.x = al * s0 + kq * u2.x;
      o2.y = al * s1 + kq * u2.y;
      const int own = (a.t - 1) * a.B_max + b0 + bb;
      *reinterpret_cast<f32x2_t*>(a.rec_u + (arena + own) * d_v + dvi) = u2;
      *reinterpret_cast<f32x2_t*>(a.o + row * d_v + dvi) = o2;
    }
  }
}

bool fused_supported(int d_k, int d_v, int L_max) {
  return d_k == kDK && d_v % 32 == 0 && d_v >= 32 && d_v <= 256 && fused_lds_bytes(16, L_max) <= 160 * 1024;
}

size_t fused_lds_bytes(int tile, int L_max) { return (size_t)fused_layout(tile, L_max).total; }

int fused_pick_tile(int R, int H, int n, int d_v, int L_max, int requested) {
  (void)d_v;
  if (requested) return requested;
  const long G = (long)R * H;
  const int cands[3] = {64, 32, 16};
  for (int c : cands) {
    const long wgs = G * ((n + c - 1) / c);
    if (wgs >= 1024 && fused_lds_bytes(c, L_max) <= 64 * 1024) return c;
  }
  return 16;
}

hipError_t launch_step_fused(const StepArgs& a, int tile, hipStream_t s) {
  const int ntile = (a.n + tile - 1) / tile;
  dim3 grid((unsigned)((size_t)a.R * a.H * ntile)), block(2 * a.d_v);
  const size_t lds = fused_lds_bytes(tile, a.L_max);
#define ONELA_FUSED_CASE(NB)                                                                                   \
  case NB:                                                                                                     \
    if (lds > 64 * 1024) {                                                                                     \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&step_fused_kernel<NB>),                \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);               \
      if (e != hipSuccess) return e;                                                                           \
    }                                                                                                          \
    hipLaunchKernelGGL(step_fused_kernel<NB>, grid, block, lds, s, a, ntile);                                  \
    break;
  switch (tile) {
    ONELA_FUSED_CASE(16)
    ONELA_FUSED_CASE(32)
    ONELA_FUSED_CASE(64)
    ONELA_FUSED_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef ONELA_FUSED_CASE
  return hipGetLastError();
}

}  // namespace onela
