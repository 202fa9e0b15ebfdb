// Chunked GDN prefill on the matrix cores (gfx950), for d_k = 128 and d_v in {16, 32, 64, 128, 256}.
//
// The recurrence is the gated delta rule of Gated DeltaNet (paper index page, "Builds on"), from the zero
// state, producing the shared post-prefill state S_ctx ("Scientific Impact Assessment: OneLA", §1):
//   u_i = beta_i (v_i - alpha_i S_{i-1} k_i),  S_i = alpha_i S_{i-1} + u_i k_i^T.
// Over a chunk of C = 32 tokens starting from S_0, with gamma_i = alpha_0 ... alpha_i, R[i][j] = alpha_{j+1} ...
// alpha_i and rc_j = R[C-1][j], unrolling the recurrence gives, exactly,
//   (I + M) U = X,  M[i][j] = beta_i R[i][j] (k_i . k_j) for j < i,  X_i = beta_i (v_i - gamma_i S_0 k_i),
//   S_C = gamma_{C-1} S_0 + sum_j rc_j u_j k_j^T,
// with U the chunk's u_i as rows.  T = (I + M)^{-1} depends on the chunk's k, alpha and beta only.  Per chunk:
//   Y = K S_0^T,  X = beta (V - gamma Y),  U = T X,  S^T <- gamma_{C-1} S^T + (diag(rc) K)^T U
// are three small matrix products, which run as v_mfma_f32_16x16x32_bf16 with every operand split into bf16
// high and low halves (a b ~ a_h b_h + a_h b_l + a_l b_h, float32 accumulation).  The decays are running
// products (no quotient of prefix products), so alpha = 0 needs no special case.
//
// Two kernels, run per segment of chunks (a segment is as many chunks as the scratch holds for every
// (request, head); usually the whole prompt):
//   prefill_t_kernel  T depends on the chunk's k, alpha and beta only, so every chunk's T is formed in
//            parallel, one wave per chunk: G = K K^T on MFMA with k read from HBM, M, the two 16 x 16 diagonal
//            blocks of T by forward substitution and the off-diagonal block as -D M21 A, in a 32 x 32 LDS
//            scratch per wave.  T's MFMA operands (bf16 high/low, in lane order), gamma, rc and beta go to
//            the scratch in HBM.
//   prefill_mfma_kernel  the chunk chain.  Workgroup = one (request, head) and a block of DV = min(d_v, 128)
//            columns of S^T (the state transposed, d_k x d_v; the columns are independent given T), DV / 16
//            waves.  Wave w holds columns 16w .. 16w+15 of the block in registers as 8 accumulator tiles of
//            16 x 16: lane l = 16 g + c holds S^T[16 n + 4 g + e][16 w + c], n = 0..7, e = 0..3.  Within each
//            32-long contraction the MFMA's k slot 8 g + j of lane l stands for index 4 g + j (j < 4) or
//            16 + 4 g + j - 4 (j >= 4) of the 32: that is exactly which of its own accumulator values a lane
//            holds, so S^T, X and U feed the next product without moving between lanes; the matching operands
//            are read from LDS in the same order.  Per chunk: T's operands, gamma, rc, beta, v, the k rows
//            (bf16 high/low) and float32 k go to LDS (fetched one chunk ahead into registers), then k scaled
//            by rc is transposed in LDS, then every wave runs its three products.  The state enters from and
//            leaves to sctx_t between segments.
// Tokens past the end pad with k = 0, v = 0, alpha = 1, beta = 0: a token that leaves the state unchanged.
#include <algorithm>

#include "device_common.h"
#include "launchers.h"

namespace onela {

namespace {
constexpr int kC = 32;      // tokens per chunk
constexpr int kDK = 128;    // d_k of this kernel
constexpr int kTWaves = 4;  // chunks (waves) per workgroup of the T-forming kernel
constexpr int kKRow = 136;  // bf16 per row of the K rows (128 + 8 padding)
constexpr int kFRow = 132;  // floats per row of the float32 K rows
constexpr int kTRow = 36;   // bf16 per row of the transposed K rows (32 + 4 padding)
constexpr int kGRow = 36;   // floats per row of a wave's 32 x 32 scratch
// bytes of T's MFMA operands per chunk: 2 row blocks x 64 lanes x (16 bytes high, 16 bytes low)
constexpr int kTOp = 2 * 64 * 32;
// scratch bytes per chunk and (request, head): T's operands, then gamma, rc and beta (3 x 32 floats)
constexpr int kChunkBytes = kTOp + 3 * kC * 4;

struct PmLds {
  int top, gs, kh, kl, kf, kth, ktl, v, vrow, total;
};

// The current chunk's T operands and gamma, rc, beta [3][32]; K rows (bf16 high, low; float32), (rc K)^T rows
// (bf16 high, low) and V rows (float32).
__host__ __device__ inline PmLds pm_layout(int d_v) {
  PmLds l;
  int off = 0;
  l.top = off;   off += kTOp;
  l.gs = off;    off += 3 * kC * 4;
  l.kh = off;    off += kC * kKRow * 2;
  l.kl = off;    off += kC * kKRow * 2;
  l.kf = off;    off += kC * kFRow * 4;
  l.kth = off;   off += kDK * kTRow * 2;
  l.ktl = off;   off += kDK * kTRow * 2;
  l.vrow = d_v + 4;
  l.v = off;     off += kC * l.vrow * 4;
  l.total = off;
  return l;
}

// (a, b) -> bf16 pairs of the high halves RNE(a), RNE(b) and the low halves RNE(a - RNE(a)), RNE(b - RNE(b))
// (the differences are exact in float32), element a in the low 16 bits; v_cvt_pk_bf16_f32 rounds to
// nearest even
__device__ __forceinline__ void split2(float a, float b, uint32_t& h, uint32_t& l) {
  const f32x2_t x = {a, b};
  const bf16x2_t hb = __builtin_convertvector(x, bf16x2_t);
  const f32x2_t hf = __builtin_convertvector(hb, f32x2_t);
  h = __builtin_bit_cast(uint32_t, hb);
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - hf, bf16x2_t));
}

// 8 floats -> bf16x8 high and low halves, element j at bits 16 (j % 2) of dword j / 2
__device__ __forceinline__ void split8(const float (&x)[8], u32x4_t& h, u32x4_t& l) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t hp, lp;
    split2(x[2 * p], x[2 * p + 1], hp, lp);
    h[p] = hp;
    l[p] = lp;
  }
}

// The operand of lane (g, m) for one 32-long contraction from bf16 rows in LDS: elements 4g .. 4g+3 and
// 16 + 4g .. 16 + 4g + 3 of the row (base at the 32-long slice)
__device__ __forceinline__ bf16x8_t lds_operand(const uint16_t* row, int g) {
  const uint2 a = *reinterpret_cast<const uint2*>(row + 4 * g);
  const uint2 b = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8_t, (u32x4_t){a.x, a.y, b.x, b.y});
}

__device__ __forceinline__ floatx4_t mfma3(bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl, floatx4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }
}  // namespace

// One wave per chunk x0 + xl of (request, head) rh: T's operands, gamma, rc and beta to the scratch slot
// (rh, xl).
__global__ __launch_bounds__(64 * kTWaves) void prefill_t_kernel(const float* __restrict__ kin,
                                                                 const float* __restrict__ ain,
                                                                 const float* __restrict__ bin, int H, int N, int x0,
                                                                 int nseg, unsigned char* __restrict__ scratch) {
  __shared__ __align__(16) float scr_all[kTWaves * kC * kGRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rh = blockIdx.x, xl = blockIdx.y * kTWaves + wave;
  if (xl >= nseg) return;  // whole waves only: nothing below synchronises the workgroup
  const int r = rh / H, h = rh - r * H, x = x0 + xl;
  const int g = lane >> 4, c = lane & 15;
  const size_t tok0 = (size_t)r * N * H + h;  // token n of this (request, head): row tok0 + n * H
  float* scr = scr_all + wave * kC * kGRow;
  unsigned char* out = scratch + ((size_t)rh * nseg + xl) * kChunkBytes;

  // alpha and beta of the chunk (lane l < 32: token l), gamma and rc by scans over the 32 lanes
  const int nl = x * kC + (lane & 31);
  const bool live = lane < kC && nl < N;
  const float al = live ? ain[tok0 + (size_t)nl * H] : 1.f;
  const float be = live ? bin[tok0 + (size_t)nl * H] : 0.f;
  float gp = lane < kC ? al : 1.f;
  float sp = __shfl_down(gp, 1, 64);
  if (lane + 1 >= kC) sp = 1.f;
#pragma unroll
  for (int off = 1; off < kC; off <<= 1) {
    const float a = __shfl_up(gp, off, 64), b = __shfl_down(sp, off, 64);
    if (lane >= off) gp *= a;
    if (lane + off < kC) sp *= b;
  }
  float* gs = reinterpret_cast<float*>(out + kTOp);
  if (lane < kC) {
    gs[lane] = gp;
    gs[kC + lane] = sp;
    gs[2 * kC + lane] = be;
  }
  // G = K K^T, lower blocks, with the k rows read from HBM straight into operand order
  u32x4_t kop_h[2][kDK / 32], kop_l[2][kDK / 32];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int n = x * kC + 16 * rb + c;
    const float* krow = kin + (tok0 + (size_t)min(n, N - 1) * H) * kDK;
#pragma unroll
    for (int s = 0; s < kDK / 32; ++s) {
      f32x4_t a = *reinterpret_cast<const f32x4_t*>(krow + 32 * s + 4 * g);
      f32x4_t b = *reinterpret_cast<const f32x4_t*>(krow + 32 * s + 16 + 4 * g);
      if (n >= N) a = b = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      const float v8[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      split8(v8, kop_h[rb][s], kop_l[rb][s]);
    }
  }
#pragma unroll
  for (int blk = 0; blk < 3; ++blk) {  // (ib, jb) = (0, 0), (1, 0), (1, 1)
    const int ib = blk == 0 ? 0 : 1, jb = blk == 2 ? 1 : 0;
    floatx4_t acc = (floatx4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kDK / 32; ++s)
      acc = mfma3(as_bf16x8(kop_h[ib][s]), as_bf16x8(kop_l[ib][s]), as_bf16x8(kop_h[jb][s]), as_bf16x8(kop_l[jb][s]),
                  acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) scr[(16 * ib + 4 * g + e) * kGRow + 16 * jb + c] = acc[e];
  }
  // M[i][j] = beta_i R[i][j] G[i][j] (j < i), R[i][j] = alpha_{j+1} .. alpha_i as a running product
  {
    const int i = lane & 31;
    const float bi = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * i, __float_as_int(be)));
    float grow[kC];
#pragma unroll
    for (int j4 = 0; j4 < kC; j4 += 4) {
      const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(scr + i * kGRow + j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) grow[j4 + e] = q4[e];
    }
    float rr = 1.f;
#pragma unroll
    for (int j = kC - 2; j >= 0; --j) {
      const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), j + 1));
      if (j < i) {
        rr *= a1;
        grow[j] = bi * rr * grow[j];
      }
    }
    if (lane < kC) {
#pragma unroll
      for (int j4 = 0; j4 < kC; j4 += 4)
        *reinterpret_cast<f32x4_t*>(scr + i * kGRow + j4) =
            (f32x4_t){grow[j4], grow[j4 + 1], grow[j4 + 2], grow[j4 + 3]};
    }
  }
  // diagonal blocks A = (I + M11)^{-1}, D = (I + M22)^{-1}: lane j < 16 column j of A, lane 16 + j of D;
  // they overwrite M11 and M22 once every row has been read
  {
    const int j = lane & 15, o = lane & 16;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = i == j ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) acc -= scr[(o + i) * kGRow + o + m] * t[m];
      t[i] = acc;
    }
    if (lane < kC) {
#pragma unroll
      for (int i = 0; i < 16; ++i) scr[(o + i) * kGRow + o + j] = t[i];
    }
  }
  // P = M21 A into the upper-right block, then C = -D P over M21; lane (q, j): rows 4q .. 4q+3, column j
  {
    const int q = lane >> 4, j = lane & 15;
    float pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q + e;
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) acc += scr[(16 + i) * kGRow + m] * scr[m * kGRow + j];
      pv[e] = acc;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) scr[(4 * q + e) * kGRow + 16 + j] = pv[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q + e;
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) acc -= scr[(16 + i) * kGRow + 16 + m] * scr[m * kGRow + 16 + j];
      pv[e] = acc;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) scr[(16 + 4 * q + e) * kGRow + j] = pv[e];
  }
  // T's operands for U = T X: lane (g, m) of row block mb holds T[16 mb + m][4g .. 4g+3, 16 + 4g .. +3]
  // (T[i][j] = 0 for j > i: the upper-right block holds P)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int i = 16 * mb + c;
    float v8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = e < 4 ? 4 * g + e : 16 + 4 * g + e - 4;
      v8[e] = j <= i ? scr[i * kGRow + j] : 0.f;
    }
    u32x4_t th4, tl4;
    split8(v8, th4, tl4);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out) + (mb * 64 + lane) * 2;
    dst[0] = th4;
    dst[1] = tl4;
  }
}

template <int DV>  // columns of S^T per workgroup (d_v, or a 128-column block of it)
__global__ __launch_bounds__(4 * DV) __attribute__((amdgpu_waves_per_eu(DV == 128 ? 4 : 1))) void prefill_mfma_kernel(const float* __restrict__ kin,
                                                              const float* __restrict__ vin, int H, int N, int d_v,
                                                              int x0, int nseg,
                                                              const unsigned char* __restrict__ scratch,
                                                              float* __restrict__ sctx_t,
                                                              float* __restrict__ sctx_out) {
  extern __shared__ __align__(16) unsigned char pm_lds[];
  constexpr int kWaves = DV / 16;
  constexpr int kThreads = 4 * DV;
  constexpr int kKq = kC * kDK / 4 / kThreads;  // float4 pieces of k per thread per chunk
  constexpr int kVq = kC * DV / 4 / kThreads;   // float4 pieces of v per thread per chunk (= 2)
  constexpr int kTq = kTOp / 8 / kThreads;      // 8-byte pieces of T's operands per thread per chunk
  constexpr int kSq = (3 * kC + kThreads - 1) / kThreads;  // gamma / rc / beta values per thread per chunk
  static_assert(kKq >= 1 && kC * kDK / 4 % kThreads == 0 && kC * DV / 4 % kThreads == 0, "chunk split");
  static_assert(kTq >= 1 && kTOp / 8 % kThreads == 0, "T operand split");
  const PmLds lay = pm_layout(DV);
  const unsigned char* top_l = pm_lds + lay.top;
  float* gs = reinterpret_cast<float*>(pm_lds + lay.gs);  // gamma, rc, beta of the current chunk
  uint16_t* kh = reinterpret_cast<uint16_t*>(pm_lds + lay.kh);
  uint16_t* kl = reinterpret_cast<uint16_t*>(pm_lds + lay.kl);
  float* kf = reinterpret_cast<float*>(pm_lds + lay.kf);
  uint16_t* kth = reinterpret_cast<uint16_t*>(pm_lds + lay.kth);
  uint16_t* ktl = reinterpret_cast<uint16_t*>(pm_lds + lay.ktl);
  float* vs = reinterpret_cast<float*>(pm_lds + lay.v);

  const int nbk = d_v / DV, rh = blockIdx.x / nbk, cb = blockIdx.x - rh * nbk, r = rh / H, h = rh - r * H;
  const int col0 = cb * DV;  // first column of S^T (row of S) of this workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const size_t tok0 = (size_t)r * N * H + h;  // token n of this (request, head): row tok0 + n * H
  const unsigned char* sc = scratch + (size_t)rh * nseg * kChunkBytes;  // this (request, head)'s chunks

  // raw chunk data of phase B in registers, one chunk ahead
  f32x4_t kr[kKq], vr[kVq];
  uint2 tr[kTq];
  float sr[kSq];
  auto fetch = [&](int x) {  // x: global chunk index
    const unsigned char* cs = sc + (size_t)(x - x0) * kChunkBytes;
#pragma unroll
    for (int u = 0; u < kTq; ++u) tr[u] = reinterpret_cast<const uint2*>(cs)[tid + u * kThreads];
#pragma unroll
    for (int u = 0; u < kSq; ++u) {
      const int y = tid + u * kThreads;
      sr[u] = reinterpret_cast<const float*>(cs + kTOp)[y < 3 * kC ? y : 3 * kC - 1];
    }
#pragma unroll
    for (int u = 0; u < kKq; ++u) {
      const int y = tid + u * kThreads, tt = y >> 5, q = y & 31, n = x * kC + tt;
      kr[u] = n < N ? *reinterpret_cast<const f32x4_t*>(kin + (tok0 + (size_t)n * H) * kDK + 4 * q)
                    : (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kVq; ++u) {
      const int y = tid + u * kThreads, tt = y / (DV / 4), q = y - tt * (DV / 4), n = x * kC + tt;
      vr[u] = n < N ? *reinterpret_cast<const f32x4_t*>(vin + (tok0 + (size_t)n * H) * d_v + col0 + 4 * q)
                    : (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }
  };

  // S^T tiles of this wave's 16 columns: zero before the first segment, else from sctx_t
  floatx4_t St[8];
  float* dst = sctx_t + (size_t)rh * kDK * d_v;
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      St[n][e] = x0 == 0 ? 0.f : dst[(size_t)(16 * n + 4 * g + e) * d_v + col0 + 16 * wave + c];

  const int x1 = x0 + nseg;
  if (nseg > 0) fetch(x0);
  for (int x = x0; x < x1; ++x) {
    {
      // T's operands, gamma, rc, beta, v rows, k rows (bf16 high/low, float32) to LDS
#pragma unroll
      for (int u = 0; u < kTq; ++u) reinterpret_cast<uint2*>(pm_lds + lay.top)[tid + u * kThreads] = tr[u];
#pragma unroll
      for (int u = 0; u < kSq; ++u)
        if (tid + u * kThreads < 3 * kC) gs[tid + u * kThreads] = sr[u];
#pragma unroll
      for (int u = 0; u < kVq; ++u) {
        const int y = tid + u * kThreads, tt = y / (DV / 4), q = y - tt * (DV / 4);
        *reinterpret_cast<f32x4_t*>(vs + tt * lay.vrow + 4 * q) = vr[u];
      }
#pragma unroll
      for (int u = 0; u < kKq; ++u) {
        const int y = tid + u * kThreads, tt = y >> 5, q = y & 31;
        uint32_t hw[2], lw[2];
        split2(kr[u][0], kr[u][1], hw[0], lw[0]);
        split2(kr[u][2], kr[u][3], hw[1], lw[1]);
        *reinterpret_cast<uint2*>(kh + tt * kKRow + 4 * q) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2*>(kl + tt * kKRow + 4 * q) = make_uint2(lw[0], lw[1]);
        *reinterpret_cast<f32x4_t*>(kf + tt * kFRow + 4 * q) = kr[u];
      }
      if (x + 1 < x1) fetch(x + 1);  // lands during this chunk's work
      __syncthreads();
      // (rc K)^T rows: thread (column kk, tokens 4 t4 .. 4 t4 + 3), bf16 high/low, 8 bytes each
      for (int y = tid; y < kDK * (kC / 4); y += kThreads) {
        const int kk = y & (kDK - 1), t4 = y >> 7;
        float w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = gs[kC + 4 * t4 + e] * kf[(4 * t4 + e) * kFRow + kk];
        uint32_t hw[2], lw[2];
        split2(w4[0], w4[1], hw[0], lw[0]);
        split2(w4[2], w4[3], hw[1], lw[1]);
        *reinterpret_cast<uint2*>(kth + kk * kTRow + 4 * t4) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2*>(ktl + kk * kTRow + 4 * t4) = make_uint2(lw[0], lw[1]);
      }
      __syncthreads();

      // ---- Y = K S^T, X = beta (V - gamma Y), U = T X, S^T <- gamma_{C-1} S^T + (rc K)^T U ----
      floatx4_t y[2] = {(floatx4_t){0.f, 0.f, 0.f, 0.f}, (floatx4_t){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < kDK / 32; ++s) {
        const float v8[8] = {St[2 * s][0], St[2 * s][1], St[2 * s][2], St[2 * s][3],
                             St[2 * s + 1][0], St[2 * s + 1][1], St[2 * s + 1][2], St[2 * s + 1][3]};
        u32x4_t sh, sl;
        split8(v8, sh, sl);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8_t ah = lds_operand(kh + (16 * mb + c) * kKRow + 32 * s, g);
          const bf16x8_t al = lds_operand(kl + (16 * mb + c) * kKRow + 32 * s, g);
          y[mb] = mfma3(ah, al, as_bf16x8(sh), as_bf16x8(sl), y[mb]);
        }
      }
      float xv[8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * mb + 4 * g + e;
          xv[4 * mb + e] = gs[2 * kC + i] * (vs[i * lay.vrow + 16 * wave + c] - gs[i] * y[mb][e]);
        }
      u32x4_t xh, xl;
      split8(xv, xh, xl);
      float uv[8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4_t* top = reinterpret_cast<const u32x4_t*>(top_l) + (mb * 64 + lane) * 2;
        const floatx4_t u = mfma3(as_bf16x8(top[0]), as_bf16x8(top[1]), as_bf16x8(xh), as_bf16x8(xl),
                                  (floatx4_t){0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) uv[4 * mb + e] = u[e];
      }
      u32x4_t uh, ul;
      split8(uv, uh, ul);
      const float gC = gs[kC - 1];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        floatx4_t acc = St[n];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= gC;
        const bf16x8_t ah = lds_operand(kth + (16 * n + c) * kTRow, g);
        const bf16x8_t al = lds_operand(ktl + (16 * n + c) * kTRow, g);
        St[n] = mfma3(ah, al, as_bf16x8(uh), as_bf16x8(ul), acc);
      }
      __syncthreads();  // the next chunk overwrites the LDS
    }
  }

  // ---- S^T to sctx_t [d_k][d_v]; after the last segment also S to sctx_out [d_v][d_k] when requested ----
  float* so = sctx_out ? sctx_out + (size_t)rh * d_v * kDK : nullptr;
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * n + 4 * g + e, col = col0 + 16 * wave + c;
      dst[(size_t)row * d_v + col] = St[n][e];
      if (so) so[(size_t)col * kDK + row] = St[n][e];
    }
}

bool prefill_mfma_supported(int d_k, int d_v) {
  return d_k == kDK && (d_v == 16 || d_v == 32 || d_v == 64 || d_v == 128 || d_v == 256);
}

size_t prefill_mfma_chunk_bytes(int R, int H) { return (size_t)R * H * kChunkBytes; }

hipError_t launch_prefill_mfma(const float* k, const float* v, const float* alpha, const float* beta, int R, int H,
                               int N, int d_v, float* sctx_t, float* sctx_out, void* scratch, size_t scratch_bytes,
                               hipStream_t s) {
  const int nch = (N + kC - 1) / kC;
  // chunks per segment: as many as the scratch holds for every (request, head), within the grid's y limit
  const size_t fit = scratch_bytes / prefill_mfma_chunk_bytes(R, H);
  const int seg = (int)std::min<size_t>(std::min<size_t>(fit, (size_t)nch), (size_t)65535 * kTWaves);
  if (nch > 0 && seg < 1) return hipErrorInvalidValue;
  unsigned char* sc = static_cast<unsigned char*>(scratch);
  // the columns of S^T are independent given T: wide states run as 128-column workgroups sharing each T
  const int blk = d_v < 128 ? d_v : 128;
  const size_t lds = (size_t)pm_layout(blk).total;
  dim3 grid((unsigned)((size_t)R * H * (d_v / blk))), block(4 * blk);
  for (int x0 = 0;; x0 += seg) {
    const int nseg = std::min(seg, nch - x0);
    const bool last = x0 + nseg >= nch;
    if (nseg > 0) {
      hipLaunchKernelGGL(prefill_t_kernel, dim3((unsigned)(R * H), (unsigned)((nseg + kTWaves - 1) / kTWaves)),
                         dim3(64 * kTWaves), 0, s, k, alpha, beta, H, N, x0, nseg, sc);
    }
#define ONELA_PM_CASE(DV)                                                                                       \
  case DV: {                                                                                                    \
    if (lds > 64 * 1024) {                                                                                      \
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_mfma_kernel<DV>),              \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                \
      if (e != hipSuccess) return e;                                                                            \
    }                                                                                                           \
    hipLaunchKernelGGL(prefill_mfma_kernel<DV>, grid, block, lds, s, k, v, H, N, d_v, x0, nseg, sc, sctx_t,     \
                       last ? sctx_out : nullptr);                                                              \
    break;                                                                                                      \
  }
    switch (blk) {
      ONELA_PM_CASE(16)
      ONELA_PM_CASE(32)
      ONELA_PM_CASE(64)
      ONELA_PM_CASE(128)
      default:
        return hipErrorInvalidValue;
    }
#undef ONELA_PM_CASE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || last) return e;
  }
}

}  // namespace onela
