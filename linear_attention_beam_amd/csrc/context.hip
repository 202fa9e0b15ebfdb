// Ancestry index update, shared-state installation (transpose + bf16 high/low split) and GDN prefill.
#include "device_common.h"
#include "launchers.h"

namespace onela {

// ---------------------------------------------------------------------------------------------------
// Ancestry index ("Scientific Impact Assessment: OneLA", §1 item (3)): the chain of beam b after step t
// is its parent's chain for steps 1..t-1 followed by its own record slot (t-1)*B_max + b.  Only the
// index is rewritten; records stay where they were appended.  One thread per (request, beam row).
// ---------------------------------------------------------------------------------------------------
__global__ void ancestry_kernel(const int32_t* __restrict__ parent, const int32_t* __restrict__ chain_prev,
                                int32_t* __restrict__ chain_out, int R, int n, int b_prev, int B_max, int L_max,
                                int t, int* __restrict__ flag, int epoch) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= R * B_max) return;
  const int r = idx / B_max, b = idx - r * B_max;
  int32_t* out = chain_out + (size_t)idx * L_max;
  if (b >= n) {
    for (int m = 0; m < L_max; ++m) out[m] = -1;
    return;
  }
  int p = parent[(size_t)r * n + b];
  if (p < 0 || p >= b_prev) {  // reported through the sticky flag; decode as a child of beam 0
    *flag = epoch;
    p = 0;
  }
  const int32_t* src = chain_prev ? chain_prev + ((size_t)r * B_max + p) * L_max : nullptr;
  for (int m = 0; m < L_max; ++m) {
    int32_t val = -1;
    if (m < t - 1) val = src[m];
    else if (m == t - 1) val = (t - 1) * B_max + b;
    out[m] = val;
  }
}

hipError_t launch_ancestry(const int32_t* parent, const int32_t* chain_prev, int32_t* chain_out, int R, int n,
                           int b_prev, int B_max, int L_max, int t, int* flag, int epoch, hipStream_t s) {
  const int total = R * B_max;
  hipLaunchKernelGGL(ancestry_kernel, dim3((total + 255) / 256), dim3(256), 0, s, parent, chain_prev, chain_out, R,
                     n, b_prev, B_max, L_max, t, flag, epoch);
  return hipGetLastError();
}

// A fill kernel rather than a memset, so the call can sit inside a captured graph.
__global__ void clear_flag_kernel(int* flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

hipError_t launch_clear_flag(int* flag, hipStream_t s) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(64), 0, s, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// S_ctx [RH][d_v][d_k] -> S_ctx^T [RH][d_k][d_v] (float32), 32x32 tiles through LDS.
// ---------------------------------------------------------------------------------------------------
__global__ void transpose_kernel(const float* __restrict__ S, float* __restrict__ ST, int d_v, int d_k) {
  __shared__ float tile[32][33];
  const int rh = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;  // i over d_v, j over d_k
  const float* src = S + (size_t)rh * d_v * d_k;
  float* dst = ST + (size_t)rh * d_v * d_k;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int i = i0 + y, j = j0 + tx;
    tile[y][tx] = (i < d_v && j < d_k) ? src[(size_t)i * d_k + j] : 0.f;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int j = j0 + y, i = i0 + tx;
    if (i < d_v && j < d_k) dst[(size_t)j * d_v + i] = tile[tx][y];
  }
}

hipError_t launch_transpose_sctx(const float* S, float* ST, int RH, int d_v, int d_k, hipStream_t s) {
  dim3 grid((d_k + 31) / 32, (d_v + 31) / 32, RH);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, S, ST, d_v, d_k);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// bf16 high/low split of S_ctx in the operand order of the fused kernel's MFMA (A operand of
// v_mfma_f32_16x16x32_bf16: lane l holds row l%16, columns 8*(l/16)..+7 of a 16x32 block).
// Per (request, head): [hl 2][w d_v/32][ks d_k/32][mi 2][lane 64][e 8] bf16 with
//   value = S[dv = 32 w + 16 mi + lane % 16][dk = 32 ks + 8 (lane / 16) + e],
//   hi = RNE_bf16(x), lo = RNE_bf16(x - hi), so hi + lo carries 16 significant bits of x.
// One thread per 8-element fragment.
// ---------------------------------------------------------------------------------------------------
__global__ void split_frag_kernel(const float* __restrict__ ST, uint16_t* __restrict__ frag, int RH, int d_v,
                                  int d_k) {
  const int W = d_v / 32, KS = d_k / 32;
  const size_t per_rh = (size_t)W * KS * 2 * 64;  // fragments per (request, head) and per hi/lo half
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_rh * RH) return;
  const int rh = (int)(idx / per_rh);
  size_t f = idx - (size_t)rh * per_rh;
  const int lane = (int)(f & 63);
  f >>= 6;
  const int mi = (int)(f & 1);
  f >>= 1;
  const int ks = (int)(f % KS);
  const int w = (int)(f / KS);
  const int dv = 32 * w + 16 * mi + (lane & 15);
  const int dk0 = 32 * ks + 8 * (lane >> 4);
  const float* src = ST + (size_t)rh * d_k * d_v;
  uint32_t hi[8], lo[8];
  for (int e = 0; e < 8; ++e) {
    const float x = src[(size_t)(dk0 + e) * d_v + dv];
    hi[e] = f32_to_bf16_bits_rne(x);
    lo[e] = f32_to_bf16_bits_rne(x - bf16_bits_to_f32(hi[e]));
  }
  u32x4_t h4, l4;
  h4.x = hi[0] | (hi[1] << 16); h4.y = hi[2] | (hi[3] << 16); h4.z = hi[4] | (hi[5] << 16); h4.w = hi[6] | (hi[7] << 16);
  l4.x = lo[0] | (lo[1] << 16); l4.y = lo[2] | (lo[3] << 16); l4.z = lo[4] | (lo[5] << 16); l4.w = lo[6] | (lo[7] << 16);
  uint16_t* base = frag + (size_t)rh * 2 * per_rh * 8;
  const size_t off = (((size_t)w * KS + ks) * 2 + mi) * 64 + lane;
  *reinterpret_cast<u32x4_t*>(base + off * 8) = h4;
  *reinterpret_cast<u32x4_t*>(base + (per_rh + off) * 8) = l4;
}

hipError_t launch_split_frag(const float* ST, uint16_t* frag, int RH, int d_v, int d_k, hipStream_t s) {
  const size_t total = (size_t)RH * (d_v / 32) * (d_k / 32) * 2 * 64;
  hipLaunchKernelGGL(split_frag_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, ST, frag, RH, d_v,
                     d_k);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// GDN prefill from the zero state ("Scientific Impact Assessment: OneLA", §1: the shared post-prefill
// state), the gated delta rule of Gated DeltaNet (paper index page, "Builds on"):
//   p = S k,  u = beta (v - alpha p),  S <- alpha S + u k^T.
// Row i of S evolves on its own: it needs v_i and the token's shared k, alpha and beta, nothing from the
// other rows.  So the recurrence is split over rows, LANES lanes per row (4 up to d_k = 128, else 8): lane j
// of a row holds the columns of float4 groups j, j + LANES, j + 2 LANES, ... of d_k (padded with zero columns
// to a multiple of 32) in registers, and p is summed over the row's lanes with DPP, with no barrier per
// token.  A workgroup of 128 LANES threads takes 128 rows of one (request, head).  Tokens come in blocks of
// kPfT: k, the workgroup's v entries, alpha and beta of a block are staged in LDS (two buffers, one barrier
// per block), fetched from HBM into registers one block ahead.
// The decay is carried as a scale, S = g Ŝ with g the running product of alpha: a token then costs one
// FMA per element for the update, Ŝ += (u / g) k^T.  When g falls below 2^-20 (also when alpha = 0) it
// is folded into Ŝ and reset to 1.
// ---------------------------------------------------------------------------------------------------
namespace {
constexpr int kPfT = 16;                 // tokens per staged block
constexpr int kPfRows = 128;             // rows of S per workgroup
constexpr float kPfRenorm = 0x1p-20f;
}  // namespace

// Lanes per row of S for d_k padded to 32 * per4 columns: 4 up to d_k = 128 (32 state columns per lane; fewer
// lanes per row mean fewer DPP steps and LDS reads per FMA), 8 above (the register state would not fit).
constexpr int prefill_lanes(int per4) { return per4 <= 4 ? 4 : 8; }

// LDS per buffer: k [kPfT][d_kp], v [kPfT][kPfRows], alpha and beta [kPfT]
inline size_t prefill_lds_bytes(int d_kp) { return 2 * (size_t)(kPfT * (d_kp + kPfRows + 2)) * sizeof(float); }

template <int PER4, int LANES>  // d_k padded to 32 * PER4 columns; LANES lanes per row of S
__global__ __launch_bounds__(LANES * kPfRows) void prefill_kernel(const float* __restrict__ kin,
                                                             const float* __restrict__ vin,
                                                             const float* __restrict__ ain,
                                                             const float* __restrict__ bin, int H, int N, int d_k,
                                                             int d_v, int nrb, float* __restrict__ sctx_t,
                                                             float* __restrict__ sctx_out) {
  extern __shared__ __align__(16) float pf_lds[];
  constexpr int kPfLanes = LANES, kPfThreads = LANES * kPfRows;
  constexpr int d_kp = 32 * PER4;
  constexpr int buf_floats = kPfT * (d_kp + kPfRows + 2);
  constexpr int kLd = (kPfT * d_kp + kPfThreads - 1) / kPfThreads;  // staged k elements per thread
  constexpr int vLd = kPfT * kPfRows / kPfThreads;                  // staged v elements per thread
  const int rh = blockIdx.x / nrb, rb = blockIdx.x - rh * nrb;
  const int r = rh / H, h = rh - r * H;
  const int tid = threadIdx.x;
  const int row = tid / kPfLanes, j = tid % kPfLanes;
  const int i = rb * kPfRows + row;  // this lane's row of S (beyond d_v: computed on zeros, not stored)
  const size_t tok0 = (size_t)r * N * H + h;  // token n of this (request, head): index tok0 + n * H

  float kr[kLd], vr[vLd], abr = 0.f;
  auto fetch = [&](int blk) {  // block blk of tokens into registers (zeros past N, past d_k, past d_v)
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int x = tid + u * kPfThreads, tt = x / d_kp, c = x - tt * d_kp, n = blk * kPfT + tt;
      kr[u] = (x < kPfT * d_kp && c < d_k && n < N) ? kin[(tok0 + (size_t)n * H) * d_k + c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < vLd; ++u) {
      const int x = tid + u * kPfThreads, tt = x / kPfRows, c = x - tt * kPfRows, n = blk * kPfT + tt;
      const int iv = rb * kPfRows + c;
      vr[u] = (iv < d_v && n < N) ? vin[(tok0 + (size_t)n * H) * d_v + iv] : 0.f;
    }
    if (tid < 2 * kPfT) {
      const int n = blk * kPfT + (tid >> 1);
      abr = n < N ? ((tid & 1) ? bin : ain)[tok0 + (size_t)n * H] : 0.f;
    }
  };
  auto stage = [&](int buf) {
    float* base = pf_lds + buf * buf_floats;
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int x = tid + u * kPfThreads;
      if (x < kPfT * d_kp) base[x] = kr[u];
    }
#pragma unroll
    for (int u = 0; u < vLd; ++u) base[kPfT * d_kp + tid + u * kPfThreads] = vr[u];
    if (tid < 2 * kPfT) base[kPfT * (d_kp + kPfRows) + tid] = abr;  // (alpha, beta) pairs per token
  };

  constexpr int kG = 8 * PER4 / kPfLanes;  // float4 column groups per lane
  float S[4 * kG];
#pragma unroll
  for (int e = 0; e < 4 * kG; ++e) S[e] = 0.f;
  float g = 1.f;  // S = g * (the registers)
  const int nblk = (N + kPfT - 1) / kPfT;
  if (nblk > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    if (blk + 1 < nblk) fetch(blk + 1);
    const float* kb = pf_lds + buf * buf_floats;
    const float* vb = kb + kPfT * d_kp;
    const float* ab = vb + kPfT * kPfRows;
    const int ntok = min(kPfT, N - blk * kPfT);
    for (int tt = 0; tt < ntok; ++tt) {
      f32x4_t kk[kG];
#pragma unroll
      for (int m = 0; m < kG; ++m) kk[m] = *reinterpret_cast<const f32x4_t*>(kb + tt * d_kp + 4 * (j + kPfLanes * m));
      const float vi = vb[tt * kPfRows + row];
      const f32x2_t a_b = *reinterpret_cast<const f32x2_t*>(ab + 2 * tt);
      f32x4_t acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < kG; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += S[4 * m + e] * kk[m][e];
      float dot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      // sum over the row's lanes: swap neighbours, swap pairs (then, for 8 lanes, mirror within the half row)
      dot += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dot), 0xB1, 0xF, 0xF, true));
      dot += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dot), 0x4E, 0xF, 0xF, true));
      if constexpr (kPfLanes == 8)
        dot += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(dot), 0x141, 0xF, 0xF, true));
      const float alpha = a_b.x, beta = a_b.y;
      const float u = beta * (vi - alpha * (g * dot));
      float gn = alpha * g;
      if (gn < kPfRenorm) {  // the same decision in every lane (alpha and g are shared)
#pragma unroll
        for (int e = 0; e < 4 * kG; ++e) S[e] *= gn;
        gn = 1.f;
      }
      const float c = u * __builtin_amdgcn_rcpf(gn);
#pragma unroll
      for (int m = 0; m < kG; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[4 * m + e] += c * kk[m][e];
      g = gn;
    }
    if (blk + 1 < nblk) stage(buf ^ 1);
    __syncthreads();
  }
  if (i < d_v) {
    float* dst = sctx_t + (size_t)rh * d_k * d_v;
    float* so = sctx_out ? sctx_out + ((size_t)rh * d_v + i) * d_k : nullptr;
#pragma unroll
    for (int m = 0; m < kG; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 4 * (j + kPfLanes * m) + e;
        if (col < d_k) {
          const float x = g * S[4 * m + e];
          dst[(size_t)col * d_v + i] = x;
          if (so) so[col] = x;
        }
      }
  }
}

bool prefill_supported(int d_k, int d_v) { return d_k >= 1 && d_k <= 256 && d_v >= 1 && d_v <= 256; }

hipError_t launch_prefill(const float* k, const float* v, const float* alpha, const float* beta, int R, int H,
                          int N, int d_k, int d_v, float* sctx_t, float* sctx_out, void* scratch,
                          size_t scratch_bytes, hipStream_t s) {
  if (prefill_mfma_supported(d_k, d_v) && (N == 0 || scratch_bytes >= prefill_mfma_chunk_bytes(R, H)))
    return launch_prefill_mfma(k, v, alpha, beta, R, H, N, d_v, sctx_t, sctx_out, scratch, scratch_bytes, s);
  const int per4 = (d_k + 31) / 32;
  const int nrb = (d_v + kPfRows - 1) / kPfRows;
  const size_t lds = prefill_lds_bytes(32 * per4);
  dim3 grid((unsigned)((size_t)R * H * nrb)), block(prefill_lanes(per4) * kPfRows);
#define ONELA_PREFILL_CASE(P)                                                                                  \
  case P:                                                                                                      \
    if (lds > 64 * 1024) {                                                                                     \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<P, prefill_lanes(P)>), \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);               \
      if (e != hipSuccess) return e;                                                                           \
    }                                                                                                          \
    hipLaunchKernelGGL((prefill_kernel<P, prefill_lanes(P)>), grid, block, lds, s, k, v, alpha, beta, H, N, d_k, \
                       d_v, nrb, sctx_t, sctx_out);                                                            \
    break;
  switch (per4) {
    ONELA_PREFILL_CASE(1)
    ONELA_PREFILL_CASE(2)
    ONELA_PREFILL_CASE(3)
    ONELA_PREFILL_CASE(4)
    ONELA_PREFILL_CASE(5)
    ONELA_PREFILL_CASE(6)
    ONELA_PREFILL_CASE(7)
    ONELA_PREFILL_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef ONELA_PREFILL_CASE
  return hipGetLastError();
}

}  // namespace onela
