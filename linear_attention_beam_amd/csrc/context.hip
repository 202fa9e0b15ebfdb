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
// One workgroup of 256 threads per (request, head) keeps S^T in registers: thread (i, part) owns column
// i of S^T (row i of S) for d_k / NPART consecutive keys, NPART = 256 / d_v.  Token inputs are
// prefetched one token ahead.
// ---------------------------------------------------------------------------------------------------
template <int PER>
__global__ __launch_bounds__(256) void prefill_kernel(const float* __restrict__ kin, const float* __restrict__ vin,
                                                      const float* __restrict__ ain, const float* __restrict__ bin,
                                                      int H, int N, int d_k, int d_v, float* __restrict__ sctx_t,
                                                      float* __restrict__ sctx_out) {
  __shared__ float sk[2][256];
  __shared__ float sv[2][256];
  __shared__ float sab[2][2];
  __shared__ float part_sum[256];
  const int rh = blockIdx.x;
  const int r = rh / H, h = rh - r * H;
  const int tid = threadIdx.x;
  const int nparts = 256 / d_v;
  const int i = tid % d_v, part = tid / d_v;
  const int d0 = part * PER;
  float st[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) st[j] = 0.f;

  auto tok_k = [&](int n) { return kin + (((size_t)r * N + n) * H + h) * d_k; };
  auto tok_v = [&](int n) { return vin + (((size_t)r * N + n) * H + h) * d_v; };
  auto tok_s = [&](int n) { return ((size_t)r * N + n) * H + h; };
  float nk = 0.f, nv = 0.f, na = 0.f, nb = 0.f;
  if (N > 0) {
    if (tid < d_k) nk = tok_k(0)[tid];
    if (tid < d_v) nv = tok_v(0)[tid];
    if (tid == 0) { na = ain[tok_s(0)]; nb = bin[tok_s(0)]; }
  }
  for (int n = 0; n < N; ++n) {
    const int buf = n & 1;
    if (tid < d_k) sk[buf][tid] = nk;
    if (tid < d_v) sv[buf][tid] = nv;
    if (tid == 0) { sab[buf][0] = na; sab[buf][1] = nb; }
    __syncthreads();
    if (n + 1 < N) {  // prefetch the next token while this one is processed
      if (tid < d_k) nk = tok_k(n + 1)[tid];
      if (tid < d_v) nv = tok_v(n + 1)[tid];
      if (tid == 0) { na = ain[tok_s(n + 1)]; nb = bin[tok_s(n + 1)]; }
    }
    float p = 0.f;
    if (part < nparts) {
#pragma unroll
      for (int j = 0; j < PER; ++j) p += st[j] * sk[buf][d0 + j];
    }
    part_sum[tid] = p;
    __syncthreads();
    if (part < nparts) {
      float pi = 0.f;
      for (int q = 0; q < nparts; ++q) pi += part_sum[q * d_v + i];
      const float a = sab[buf][0], b = sab[buf][1];
      const float u = b * (sv[buf][i] - a * pi);
#pragma unroll
      for (int j = 0; j < PER; ++j) st[j] = a * st[j] + u * sk[buf][d0 + j];
    }
    // part_sum is rewritten only after the next barrier; sk/sv/sab alternate buffers.
  }
  if (part < nparts) {
    float* dst = sctx_t + (size_t)rh * d_k * d_v;
#pragma unroll
    for (int j = 0; j < PER; ++j) dst[(size_t)(d0 + j) * d_v + i] = st[j];
    if (sctx_out) {
      float* so = sctx_out + (size_t)rh * d_v * d_k + (size_t)i * d_k + d0;
#pragma unroll
      for (int j = 0; j < PER; ++j) so[j] = st[j];
    }
  }
}

bool prefill_supported(int d_k, int d_v) {
  if (d_v < 1 || d_v > 256 || 256 % d_v != 0) return false;
  const int nparts = 256 / d_v;
  if (d_k < 1 || d_k > 256 || d_k % nparts != 0) return false;
  const int per = d_k / nparts;
  return per <= 128 && (per & (per - 1)) == 0;
}

hipError_t launch_prefill(const float* k, const float* v, const float* alpha, const float* beta, int R, int H,
                          int N, int d_k, int d_v, float* sctx_t, float* sctx_out, hipStream_t s) {
  const int per = d_k / (256 / d_v);
  dim3 grid(R * H), block(256);
#define ONELA_PREFILL_CASE(P)                                                                                  \
  case P:                                                                                                      \
    hipLaunchKernelGGL(prefill_kernel<P>, grid, block, 0, s, k, v, alpha, beta, H, N, d_k, d_v, sctx_t,       \
                       sctx_out);                                                                              \
    break;
  switch (per) {
    ONELA_PREFILL_CASE(1)
    ONELA_PREFILL_CASE(2)
    ONELA_PREFILL_CASE(4)
    ONELA_PREFILL_CASE(8)
    ONELA_PREFILL_CASE(16)
    ONELA_PREFILL_CASE(32)
    ONELA_PREFILL_CASE(64)
    ONELA_PREFILL_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef ONELA_PREFILL_CASE
  return hipGetLastError();
}

}  // namespace onela
