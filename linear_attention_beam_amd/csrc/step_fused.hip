// Fused projection-replay decode step for gfx950 ("Scientific Impact Assessment: OneLA", §1: a fused GPU
// kernel reuses S_ctx across beams; paper index page, Abstract).  Two launches per step (one at step 1):
//
// ancestry_plan_kernel (steps t >= 2), one workgroup per request.
//   * The ancestry index (review §1 item (3)): each beam's chain is its parent's chain from the previous table
//     plus its own slot; the kernel writes the new table.
//   * A processing order: the beams sorted by their history (a counting sort on the parent's place in the
//     previous step's order, which keeps the whole chains in lexicographic order).  Beams with common
//     ancestors then share tiles, so a tile touches few distinct records and neighbouring tiles share the rest.
//     The order only decides which workgroup computes which beam: every output lands at its beam's place.
//     The sort places siblings the same way in every run, so the tiles, and with them which tiles read
//     their records from memory instead of LDS (a different summation order), repeat exactly.
//   * One plan per tile of NB consecutive beams in that order, shared by every head (slots are the same for
//     all heads): the beams, the distinct ancestor slots (chain position by chain position, in order of first
//     appearance) and, for each beam and chain position, the place of its record in that list.
//
// step_fused_kernel, persistent: a workgroup walks a list of jobs (request, head, block of RB rows of d_v, run
//   of beam tiles); two workgroups share a compute unit.  Wavefront w owns d_v rows RB*rb + 16w .. +15 of
//   S_ctx, whose bf16 high and low halves stay in registers for the whole job (S_ctx is read once per job and
//   reused by every beam of every tile of the job).  Per tile:
//   * one round trip brings everything into LDS: the beams' k, q and v rows (16-byte loads through registers),
//     and, copied straight into LDS (global_load_lds), the keys, alphas and u rows of the tile's distinct
//     ancestor records, the beams and the plan places, all issued at a raised wave priority.  The plan itself
//     was loaded during the previous tile;
//   * the dot products of every staged record key with every beam's k and q on the matrix cores (16 records x
//     16 beams per output tile); then one thread per beam walks its chain newest to oldest, scaling them by the
//     decay product c_j of the alphas after record j;
//   * per 16 beams, v_mfma_f32_16x16x32_bf16 forms [P_k | P_q]^T = S_rows [k | q], high then low half into one
//     float32 accumulator; in the accumulator lane l holds beam l % 16 and d_v rows 4 (l / 16) .. +3 of the
//     wavefront's 16 rows, so the replay works per beam on 16-byte pieces of u, and u and o leave as float4:
//       p = A P_k + sum_j c_j (K_j . k) U_j,   u = beta (v - alpha p),
//       o = alpha (A P_q + sum_j c_j (K_j . q) U_j) + (k . q) u,        A = prod_j alpha_j.
//   A tile whose distinct records do not fit in LDS reads them from memory instead: d_k / 8 lanes per beam take
//   the key dot products (a different summation order from the matrix cores') and the replay reads u from memory.
//   The kernel is built for d_k = 64, 128 and 256 (d_k / 32 matrix-core k-steps, rows of d_k / 8 pieces); at
//   d_k = 256 the S_ctx rows take 64 registers per wavefront and one workgroup runs per compute unit.
#include <algorithm>

#include "device_common.h"
#include "launchers.h"

namespace onela {

namespace {
constexpr int kCap = 64;        // distinct ancestor records of a tile staged in LDS (beyond: read from memory)
constexpr int kSort = 2048;     // beams per request the plan kernel sorts (more: they keep their own order)

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }
// A k or q row of d_k = DK bf16 values is DK / 8 pieces of 16 bytes.  Piece p of row (or record) i of a tile in
// LDS holds chunk p ^ ONELA_SWZ(i): the 16 rows that one matrix-core operand read touches at one chunk fall in
// different banks (rows of 256 or 512 bytes at d_k = 128 or 256: 16 chunks of one 256-byte span; two rows of 128
// bytes per 256 at d_k = 64).  A macro, so that the compiler sees the plain mask where it folds the surrounding
// index arithmetic.
#define ONELA_SWZ(i) (DK >= 128 ? ((i) & 15) : (((i) >> 1) & 7))
// Bytes per beam of the record places (one per chain position): a multiple of 8, so that the replay reads a
// beam's places eight at a time.
__host__ __device__ inline int li_stride(int L) { return (L + 7) & ~7; }

// Plan record of one (request, tile), in bytes: nd, the distinct slots (up to kCap), the NB beams (padded with
// the last beam), then one byte per (beam, chain position): the place of its record in the distinct list.
struct PlanLayout {
  int perm, li, bytes;
};
__host__ __device__ inline PlanLayout plan_layout(int NB, int L) {
  PlanLayout p;
  p.perm = align16(4 + 4 * kCap);
  p.li = p.perm + NB * 4;
  p.bytes = p.li + align16(NB * li_stride(L));
  return p;
}

// LDS layout of one tile.
struct FusedLds {
  int xk, xq, xv, al, be, pm, li, kd, ud, ad, coef, beamA, beamKq, total;
};
// Coefficients per beam: room for the chain rounded up to four positions (those past the chain hold zeros),
// odd so that 16 beams fall in distinct banks.
__host__ __device__ inline int coef_stride(int L) { return ((L + 3) & ~3) | 1; }
__host__ __device__ inline FusedLds fused_layout(int NB, int L, int RB, int DK) {
  FusedLds y;
  const int kRow = 2 * DK;  // bytes per k or q row (bf16)
  int o = 0;
  y.xk = o;  o += NB * kRow;               // k rows, 16-byte pieces swizzled by row
  y.xq = o;  o += NB * kRow;               // q rows
  y.xv = o;  o += NB * RB * 2;             // this row block of the v rows, swizzled
  y.al = o;  o += align16(NB * 4);
  y.be = o;  o += align16(NB * 4);
  y.pm = o;  o += align16(NB * 4);         // the tile's beams
  y.li = o;  o += align16(NB * li_stride(L));  // place of each chain record in the distinct list
  y.kd = o;  o += std::max(kCap * kRow, kCap * NB * 8);  // keys of the distinct records, then their dot products
  y.ud = o;  o += kCap * RB * 4;           // their u rows of this row block, 16-byte pieces swizzled by record
  y.ad = o;  o += align16(kCap * 4);       // their alphas at this head
  y.coef = o;   o += NB * coef_stride(L) * 8;
  y.beamA = o;  o += align16(NB * 4);
  y.beamKq = o; o += align16(NB * 4);
  y.total = o;
  return y;
}

// Rows of d_v per job: the largest of 128, 64, 32 that divides d_v.
__host__ __device__ inline int row_block(int d_v) { return d_v % 128 == 0 ? 128 : (d_v % 64 == 0 ? 64 : 32); }

// Job schedule: job j = (request, head, row block, run of tiles).  Jobs of one (request, head) are congruent
// modulo 8, so with a grid that is a multiple of 8 they run on one XCD (dispatch is round-robin over 8) and
// share its L2 for the head's records.
struct Sched {
  int RH, NRB, ntile, TJ, JPR, njobs;
};
inline Sched make_sched(int RH, int NRB, int ntile, int grid) {
  Sched s;
  s.RH = RH;
  s.NRB = NRB;
  s.ntile = ntile;
  const long total = (long)RH * NRB * ntile;
  s.TJ = (int)std::max(1L, std::min((long)ntile, total / std::max(grid, 1)));
  s.JPR = (ntile + s.TJ - 1) / s.TJ;
  s.njobs = RH * NRB * s.JPR;
  return s;
}
struct Job {
  int rh, rb, t0, t1;
};
__device__ inline Job job_of(const Sched& s, int j) {
  Job q;
  int rem;
  const int per = s.NRB * s.JPR;
  if ((s.RH & 7) == 0) {
    const int x = j & 7, y = j >> 3;
    // group g = y / per holds (request, head) pairs 8g .. 8g + 7; XCD x takes pair 8g + ((x + g) mod 8), so
    // that each XCD serves every head residue over the groups: the heads' rows sit at fixed offsets in the
    // beam-major inputs, and with a fixed residue per XCD two of the eight XCDs were 5% slower
    q.rh = (y / per) * 8 + ((x + y / per) & 7);
    rem = y - (y / per) * per;
  } else {
    q.rh = j / per;
    rem = j - q.rh * per;
  }
  q.rb = rem / s.JPR;
  const int jr = rem - q.rb * s.JPR;
  q.t0 = jr * s.TJ;
  q.t1 = min(s.ntile, q.t0 + s.TJ);
  return q;
}

// Cursor over a workgroup's (job, tile) sequence.
struct Cursor {
  int job, tile;
  Job J;
  bool valid;
};
__device__ inline Cursor cursor_first(const Sched& s) {
  Cursor c;
  c.job = blockIdx.x;
  c.valid = c.job < s.njobs;
  c.tile = 0;
  if (c.valid) {
    c.J = job_of(s, c.job);
    c.tile = c.J.t0;
  }
  return c;
}
__device__ inline Cursor cursor_next(const Sched& s, Cursor c) {
  if (!c.valid) return c;
  if (c.tile + 1 < c.J.t1) {
    c.tile += 1;
    return c;
  }
  c.job += gridDim.x;
  c.valid = c.job < s.njobs;
  if (c.valid) {
    c.J = job_of(s, c.job);
    c.tile = c.J.t0;
  }
  return c;
}

// Copies 16 (or 4) bytes per active lane from memory straight into LDS: lane l writes dst + 16 l (4 l); dst is
// the same for the whole wavefront.
__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_dst, 4, 0, 0);
}

// Inclusive prefix sum over a wavefront.
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}
}  // namespace

// ---------------------------------------------------------------------------------------------------------
// Ancestry index, processing order and tile plans for step t >= 2 (see the top of the file).  rank[r][b]: the
// place of beam b in its request's processing order, written for the next step.
// ---------------------------------------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(1024) void ancestry_plan_kernel(StepArgs a, unsigned char* __restrict__ plan,
                                                             int plan_bytes, int perm_off, int li_off,
                                                             int* __restrict__ rank) {
  static_assert(NB <= 64, "one lane per beam of a tile");
  constexpr int kParts = 8;  // parts of the beam range, each counted and placed by one wavefront
  __shared__ int s_par[kSort];
  __shared__ int s_key[kSort];
  __shared__ int s_perm[kSort];
  __shared__ int s_tot[kSort];
  __shared__ int s_wsum[kSort / 64];
  // per part, two 16-bit counters per word: key k in half k & 1 of word k >> 1 (no count reaches 2^16)
  __shared__ unsigned s_cnt[kParts][kSort / 2];
  const int L = a.L_max, n = a.n, t = a.t, nch = t - 1;
  const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nt >> 6;
  const int ntile = (n + NB - 1) / NB;
  const bool sorted = n <= kSort && a.b_prev <= kSort && nt >= kSort / 2;
  const int* parent = a.parent + (size_t)r * n;
  auto parent_of = [&](int b) {  // range-checked: a bad index raises the sticky flag and becomes 0
    int p = parent[b];
    if (p < 0 || p >= a.b_prev) {
      *a.flag = a.epoch;
      p = 0;
    }
    return p;
  };
  if (sorted) {
    // A counting sort whose result is the same in every run: the beam range is cut into kParts parts, each
    // counted and placed by one wavefront with counters of its own, so no two wavefronts race on a counter.
    // Siblings (beams of one key) are placed part by part, within a part as its wavefront's atomics return.
    const int K = a.b_prev, C = (n + kParts - 1) / kParts;
    const int p0 = wave * C, p1 = min(n, p0 + C);
    for (int g = 0; g < kParts; ++g)
      for (int w = tid; w < (K + 1) / 2; w += nt) s_cnt[g][w] = 0u;
    __syncthreads();
    if (wave < kParts) {
      for (int b = p0 + lane; b < p1; b += 64) {
        const int p = parent_of(b);
        s_par[b] = p;
        // the parent's place in the previous step's order (step 1 has a single beam)
        const int key = nch == 1 ? p : rank[(size_t)r * a.B_max + p];
        s_key[b] = key;
        atomicAdd(&s_cnt[wave][key >> 1], 1u << (16 * (key & 1)));
      }
    }
    __syncthreads();
    {
      // Keys 2 tid and 2 tid + 1: each part's offset within the key's run, and the runs' lengths.  Then the
      // runs' exclusive offsets: a scan within each wavefront, plus the totals of the wavefronts before it.
      const int k0 = 2 * tid;
      int run0 = 0, run1 = 0;
      if (k0 < K) {
        unsigned c[kParts];
#pragma unroll
        for (int g = 0; g < kParts; ++g) c[g] = s_cnt[g][tid];
#pragma unroll
        for (int g = 0; g < kParts; ++g) {
          s_cnt[g][tid] = (unsigned)run0 | ((unsigned)run1 << 16);
          run0 += (int)(c[g] & 0xFFFFu);
          run1 += (int)(c[g] >> 16);
        }
      }
      const int pair = run0 + run1, inc = wave_scan(pair);
      if (lane == 63) s_wsum[wave] = inc;
      __syncthreads();
      // the totals of the wavefronts before this one: one per lane, summed across the wavefront
      const int before = __shfl(wave_scan(lane < wave ? s_wsum[lane] : 0), 63, 64) + inc - pair;
      if (k0 < K) s_tot[k0] = before;
      if (k0 + 1 < K) s_tot[k0 + 1] = before + run0;
    }
    __syncthreads();
    if (wave < kParts) {
      for (int b = p0 + lane; b < p1; b += 64) {
        const int k = s_key[b];
        const unsigned sh = 16u * (unsigned)(k & 1);
        const unsigned old = atomicAdd(&s_cnt[wave][k >> 1], 1u << sh);
        s_perm[s_tot[k] + (int)((old >> sh) & 0xFFFFu)] = b;
      }
    }
    __syncthreads();
    for (int pos = tid; pos < n; pos += nt) rank[(size_t)r * a.B_max + s_perm[pos]] = pos;
  } else {
    for (int b = tid; b < n; b += nt) rank[(size_t)r * a.B_max + b] = b;
  }
  // one wavefront per tile: chain rows, distinct records, plan
  for (int tile = wave; tile < ntile; tile += nwaves) {
    const int b0 = tile * NB, nb = min(NB, n - b0);
    const bool live = lane < nb;
    const int pos = b0 + min(lane, nb - 1);
    const int b = sorted ? s_perm[pos] : pos;
    const int p = sorted ? s_par[b] : parent_of(b);
    const int32_t* prow = a.chain_prev + ((size_t)r * a.B_max + p) * L;
    int32_t* out = a.chain_out + ((size_t)r * a.B_max + b) * L;
    unsigned char* rec = plan + ((size_t)r * ntile + tile) * plan_bytes;
    int* dlist = reinterpret_cast<int*>(rec + 4);
    unsigned char* li = rec + li_off;
    int base = 0;
    for (int m0 = 0; m0 < L; m0 += 8) {
      // eight chain entries of the parent's row at a time: their loads are independent
      int vv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) vv[j] = m0 + j < nch ? prow[m0 + j] : -1;
      unsigned lib[2] = {0u, 0u};  // the eight places, stored at once (one byte each)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = m0 + j;
        if (m >= L) break;
        if (m >= nch) {  // own slot, then -1
          if (live) out[m] = m == nch ? nch * a.B_max + b : -1;
          continue;
        }
        const int v = vv[j];
        if (live) out[m] = v;
        // first appearances of each record at this position (records at different positions differ: position m
        // holds slots of step m + 1).  In the sorted order the chains are in lexicographic order, and a record
        // fixes every entry before it, so the beams holding one record are adjacent: a beam is a first
        // appearance when its left neighbour holds another record.  Otherwise each lane looks for the first
        // lane with its value.
        bool is_first;
        int place;
        if (sorted) {
          const int left = __shfl_up(v, 1, 64);
          is_first = live && (lane == 0 || left != v);
          // the first appearances at or before this lane: its own record's is the last of them
          place = base + __popcll(__ballot(is_first) & ((2ull << lane) - 1ull)) - 1;
        } else {
          int o = lane;
          for (int c = nb - 1; c >= 0; --c)
            if (__builtin_amdgcn_readlane(v, c) == v) o = c;
          is_first = live && o == lane;
          place = base + __popcll(__ballot(is_first) & ((1ull << o) - 1ull));
        }
        const unsigned long long first = __ballot(is_first);
        if (is_first && place < kCap) dlist[place] = v;
        lib[j >> 2] |= (unsigned)(place & 255) << (8 * (j & 3));  // unused by the fused kernel unless nd <= kCap
        base += __popcll(first);
      }
      if (live && m0 < nch) *reinterpret_cast<u32x2_t*>(li + lane * li_stride(L) + m0) = (u32x2_t){lib[0], lib[1]};
    }
    if (lane == 0) *reinterpret_cast<int*>(rec) = base;
    if (lane < NB) reinterpret_cast<int*>(rec + perm_off)[lane] = b;
  }
  for (int idx = tid; idx < (a.B_max - n) * L; idx += nt)  // rows of beams >= n are all -1
    a.chain_out[((size_t)r * a.B_max + n) * L + idx] = -1;
}

// ---------------------------------------------------------------------------------------------------------
template <int NB, int RB, int DK>
__global__ __launch_bounds__(64 * (RB / 16), DK == 256 ? 2 : 4) void step_fused_kernel(StepArgs a, const unsigned char* __restrict__ plan,
                                                                      int plan_bytes, int perm_off, int li_off,
                                                                      Sched S) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int NW = RB / 16;      // wavefronts: wavefront w owns rows 16 w .. 16 w + 15 of the row block
  constexpr int NT = NW * 64;
  constexpr int VP = RB / 8;       // 16-byte pieces of a v row block (bf16)
  constexpr int UP = RB / 4;       // 16-byte pieces of a u row block (float32)
  constexpr int KP = DK / 8;       // 16-byte pieces of a k or q row (bf16); also lanes per beam below
  constexpr int KPL = DK == 256 ? 5 : (DK == 128 ? 4 : 3);  // log2(KP)
  constexpr int kKS = DK / 32;     // MFMA k-steps
  constexpr int kRow = 2 * DK;     // bytes per k or q row
  constexpr int KI = (kCap * KP + NT - 1) / NT;  // key pieces of the distinct records per thread
  constexpr int UI = (kCap * UP + NT - 1) / NT;  // u pieces per thread
  constexpr int NX = 2 * NB * KP + NB * VP;      // k, q and v pieces of a tile
  constexpr int XI = (NX + NT - 1) / NT;         // ... per thread
  constexpr int kTiles = NB / 16;
  const int L = a.L_max, H = a.H, n = a.n, d_v = a.d_v, t = a.t, nch = t - 1;
  const FusedLds lay = fused_layout(NB, L, RB, DK);
  const int LS = coef_stride(L), LIS = li_stride(L);
  constexpr int ngroups = NT / KP;
  const unsigned hk = (unsigned)H * DK, hv = (unsigned)H * d_v;  // beam strides of the inputs (elements)
  unsigned char* xk = lds + lay.xk;
  unsigned char* xq = lds + lay.xq;
  unsigned char* xv = lds + lay.xv;
  float* al_t = reinterpret_cast<float*>(lds + lay.al);
  float* be_t = reinterpret_cast<float*>(lds + lay.be);
  int* pm_t = reinterpret_cast<int*>(lds + lay.pm);
  const unsigned char* li_t = lds + lay.li;
  unsigned char* kd = lds + lay.kd;
  unsigned char* ud = lds + lay.ud;
  const float* ad = reinterpret_cast<const float*>(lds + lay.ad);
  f32x2_t* coef = reinterpret_cast<f32x2_t*>(lds + lay.coef);
  float* beamA = reinterpret_cast<float*>(lds + lay.beamA);
  float* beamKq = reinterpret_cast<float*>(lds + lay.beamKq);

  // What this thread needs from a tile's plan to issue the tile's loads: nd, the distinct slots of its
  // copies into LDS, and the beams of its k, q, v pieces and of its alpha and beta.  Loaded one tile ahead.
  struct Plan {
    int nd, as, ab, ks[KI], us[UI], xb[XI];
  };
  auto piece_row = [&](int q) {  // the row (place in the tile) of k, q or v piece q
    return q < 2 * NB * KP ? ((q & (NB * KP - 1)) >> KPL) : (q - 2 * NB * KP) / VP;
  };
  auto load_plan = [&](const Cursor& c, int tid) {
    Plan p;
    const int tile = c.valid ? c.tile : 0;
    const unsigned char* rec = plan + ((size_t)(c.valid ? c.J.rh / H : 0) * S.ntile + tile) * plan_bytes;
    const int* dl = reinterpret_cast<const int*>(rec + 4);
    const int* pm = reinterpret_cast<const int*>(rec + perm_off);
    p.nd = *reinterpret_cast<const int*>(rec);
#pragma unroll
    for (int i = 0; i < KI; ++i) p.ks[i] = dl[min((i * NT + tid) >> KPL, kCap - 1)];
#pragma unroll
    for (int i = 0; i < UI; ++i) p.us[i] = dl[min((i * NT + tid) / UP, kCap - 1)];
    p.as = dl[min(tid, kCap - 1)];
    p.ab = pm[min(tid, NB - 1)];
#pragma unroll
    for (int i = 0; i < XI; ++i) p.xb[i] = pm[piece_row(min(i * NT + tid, NX - 1))];
    if (nch == 0) {  // step 1 has no plan: the beams keep their order
      const int nb = min(NB, n - tile * NB);
      p.nd = 0;
      p.ab = tile * NB + min(tid, nb - 1);
#pragma unroll
      for (int i = 0; i < XI; ++i) p.xb[i] = tile * NB + min(piece_row(min(i * NT + tid, NX - 1)), nb - 1);
    }
    return p;
  };
  bf16x8_t sf[kKS][2];
  int cur_job = -1;
  Plan pl = load_plan(cursor_first(S), (int)threadIdx.x);
  __builtin_amdgcn_s_waitcnt(0);  // so that no wait for the plan is left inside the loop
  for (Cursor c = cursor_first(S); c.valid; c = cursor_next(S, c)) {
    // the thread index is laundered per tile, so that the compiler derives per-lane addresses next to their
    // use instead of keeping them live (and spilled) across the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int gq = lane >> 4, col = lane & 15;
    const int gb = tid >> KPL, jb = tid & (KP - 1);  // per-beam work: beam group, piece
    const int rh = c.J.rh, r = rh / H, h = rh - r * H, rb = c.J.rb;
    const int b0 = c.tile * NB, nb = min(NB, n - b0);
    const size_t arena = (size_t)rh * a.slots;
    const size_t rrow = (size_t)r * n * H + h;  // input row of beam 0 of this request at this head
    const float* u_rd = a.rec_u + arena * d_v;  // u arena of this (request, head): [slots][d_v]
    const unsigned char* prec = plan + ((size_t)r * S.ntile + c.tile) * plan_bytes;
    // Wave priorities order the two workgroups of a CU: the tile's global loads and its copies into LDS up to
    // the barrier run at 3 (the other workgroup is usually computing, and its waves would otherwise win the
    // issue arbitration and delay them: 7-8% per decode), the output stores at 2, the contraction and replay
    // at 1 (ahead of the other workgroup's per-beam and chain-coefficient work: 2%), the rest at 0.
    __builtin_amdgcn_s_setprio(3);
    // ---- the distinct records' keys, u rows and alphas, the beams and the plan places, copied into LDS ----
    const bool fast = nch > 0 && pl.nd <= kCap;
    const int ndl = fast ? pl.nd : 0;  // records copied into LDS
    {
      const uint16_t* kr = static_cast<const uint16_t*>(a.rec_k) + arena * DK;
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        // key piece p of distinct record d holds chunk p ^ ONELA_SWZ(d)
        const int q0 = i * NT + wave * 64, q = q0 + lane;
        if (q < ndl * KP) dma16(kr + (size_t)pl.ks[i] * DK + (((q & (KP - 1)) ^ ONELA_SWZ(q >> KPL)) << 3), kd + q0 * 16);
      }
#pragma unroll
      for (int i = 0; i < UI; ++i) {
        // u piece p of distinct record d holds row chunk p ^ (d % UP) of the row block
        const int q0 = i * NT + wave * 64, q = q0 + lane;
        const int d = q / UP, ch = (q % UP) ^ (d & (UP - 1));
        if (q < ndl * UP) dma16(u_rd + (size_t)pl.us[i] * d_v + rb * RB + 4 * ch, ud + q0 * 16);
      }
      if (wave == 0 && lane < ndl) dma4(a.rec_alpha + arena + pl.as, lds + lay.ad);
      if (nch > 0) {
        if (wave == 0 && lane < NB) dma4(prec + perm_off + lane * 4, lds + lay.pm);
        for (int q0 = wave * 64; q0 < NB * LIS / 4; q0 += NT)
          if (q0 + lane < NB * LIS / 4 && ndl > 0) dma4(prec + li_off + (q0 + lane) * 4, lds + lay.li + q0 * 4);
      }
    }
    // ---- the k, q and v rows; alpha and beta ----
    const uint16_t* kin = static_cast<const uint16_t*>(a.k) + rrow * DK;
    const uint16_t* qin = static_cast<const uint16_t*>(a.q) + rrow * DK;
    const uint16_t* vin = static_cast<const uint16_t*>(a.v) + rrow * d_v + rb * RB;
    u32x4_t X[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      // pieces 0 .. NB*KP-1: k rows, then q rows, then v rows; a k or q row's piece p holds chunk p ^ ONELA_SWZ(row),
      // a v row's chunk p ^ (row % VP)
      const int q = min(i * NT + tid, NX - 1);
      const int row = piece_row(q);
      const unsigned beam = (unsigned)pl.xb[i];
      const unsigned offk = beam * hk + (((q & (KP - 1)) ^ ONELA_SWZ(row)) << 3);
      const int qv = max(q - 2 * NB * KP, 0);
      const unsigned offv = beam * hv + (((qv % VP) ^ (row & (VP - 1))) << 3);
      const uint16_t* base = q < NB * KP ? kin : (q < 2 * NB * KP ? qin : vin);
      X[i] = *reinterpret_cast<const u32x4_t*>(base + (q < 2 * NB * KP ? offk : offv));
    }
    const float pal = a.alpha[rrow + (size_t)pl.ab * H];
    const float pbe = a.beta[rrow + (size_t)pl.ab * H];
    const int pab = pl.ab;
    pl = load_plan(cursor_next(S, c), tid);  // the next tile's plan, in flight with this tile's loads
    if (c.job != cur_job) {  // S_ctx rows of this wavefront, once per job
      cur_job = c.job;
      const int W = d_v / 32;
      const size_t half = (size_t)W * kKS * 2 * 64;
      const u32x4_t* fr = reinterpret_cast<const u32x4_t*>(a.sctx_frag) + (size_t)rh * 2 * half;
      const int x = rb * NW + wave;  // 16-row block of d_v
#pragma unroll
      for (int k2 = 0; k2 < kKS; ++k2)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
          sf[k2][hl] = __builtin_bit_cast(bf16x8_t, fr[hl * half + (((size_t)(x >> 1) * kKS + k2) * 2 + (x & 1)) * 64 + lane]);
    }
    // ---- into LDS ----
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int q = i * NT + tid;
      if (q < NX) *reinterpret_cast<u32x4_t*>(xk + q * 16) = X[i];  // the k, q and v regions are adjacent
    }
    if (tid < NB) {
      al_t[tid] = pal;
      be_t[tid] = pbe;
      if (nch == 0) pm_t[tid] = pab;
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's copies into LDS have landed
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    // ---- per beam (KP lanes): k . q, the record key and alpha; chain coefficients when read from memory ----
    for (int b = gb; b < nb; b += ngroups) {
      const int beam = pm_t[b];
      const int xo = b * kRow + ((jb ^ ONELA_SWZ(b)) << 4);
      const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(xk + xo);
      const u32x4_t qx = *reinterpret_cast<const u32x4_t*>(xq + xo);
      const float kq = rows_sum<KP>(dot8_bf16(kx, qx));
      if (!fast) {  // step 1 (no chain), or a tile whose distinct records were not staged: newest to oldest
        float cdec = 1.f;
        const int32_t* crow = a.chain_out + ((size_t)r * a.B_max + beam) * L;
        for (int m = nch - 1; m >= 0; --m) {
          const int sl = crow[m];
          const u32x4_t K = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.rec_k) + (arena + sl) * DK + jb * 8);
          const float am = a.rec_alpha[arena + sl];
          const float dk = rows_sum<KP>(dot8_bf16(K, kx));
          const float dq = rows_sum<KP>(dot8_bf16(K, qx));
          if (jb == 0) coef[b * LS + m] = (f32x2_t){cdec * dk, cdec * dq};
          cdec *= am;
        }
        if (jb == 0) beamA[b] = cdec;
      }
      if (jb == 0) beamKq[b] = kq;
      if (rb == 0) {  // the new record's key and alpha
        const unsigned own = (unsigned)(nch * a.B_max + beam);
        *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.rec_k) + (arena + own) * DK + jb * 8) = kx;
        if (jb == 0) a.rec_alpha[arena + own] = al_t[b];
      }
    }
    if (fast) {
      // Dot products of every staged record key with every beam's k and q on the matrix cores:
      // [K_D . k | K_D . q] = K_D [k | q]^T, 16 records x 16 beams per output tile, 4 k-steps of 32.  In an output
      // tile lane l holds beam l % 16 and records 4 (l / 16) .. +3; DK / 32 k-steps of 32.  Wavefront w takes
      // tiles w, w + NW, ...
      const int nrt = (ndl + 15) >> 4;
      const int ntl = nrt * kTiles * 2;
      constexpr int kMaxT = (kCap / 16) * kTiles * 2 / NW + ((kCap / 16) * kTiles * 2 % NW ? 1 : 0);
      floatx4_t dacc[kMaxT];
#pragma unroll
      for (int i = 0; i < kMaxT; ++i) {
        const int tl = wave + i * NW;
        dacc[i] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
        if (tl < ntl) {
          const int rt = tl / (kTiles * 2), rem = tl - rt * (kTiles * 2), bt = rem >> 1, kqsel = rem & 1;
          const int d = rt * 16 + col, bb = bt * 16 + col;
          const unsigned char* xs = kqsel ? xq : xk;
#pragma unroll
          for (int k2 = 0; k2 < kKS; ++k2) {
            const int ch = k2 * 4 + gq;
            const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(kd + d * kRow + ((ch ^ ONELA_SWZ(d)) << 4)));
            const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + bb * kRow + ((ch ^ ONELA_SWZ(bb)) << 4)));
            dacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, kb, dacc[i], 0, 0, 0);
          }
        }
      }
      __syncthreads();  // every wavefront is done with the staged keys: their space takes the dot products
      float* dots = reinterpret_cast<float*>(kd);  // [record][beam][k or q]
#pragma unroll
      for (int i = 0; i < kMaxT; ++i) {
        const int tl = wave + i * NW;
        if (tl < ntl) {
          const int rt = tl / (kTiles * 2), rem = tl - rt * (kTiles * 2), bt = rem >> 1, kqsel = rem & 1;
          const int bb = bt * 16 + col;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d = rt * 16 + 4 * gq + e;
            if (d < ndl) dots[(d * NB + bb) * 2 + kqsel] = dacc[i][e];
          }
        }
      }
      __syncthreads();
      // per beam, newest to oldest: c_j times the dot products, and the decay product A
      for (int b = tid; b < nb; b += NT) {
        const f32x2_t* dd = reinterpret_cast<const f32x2_t*>(dots) + b;
        float cdec = 1.f;
        for (int m = nch - 1; m >= 0; m -= 4) {
          int d[4];
          f32x2_t v[4];
          float am[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) d[j] = li_t[b * LIS + max(m - j, 0)];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = dd[d[j] * NB];
            am[j] = ad[d[j]];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (m - j >= 0) {
              coef[b * LS + m - j] = (f32x2_t){cdec * v[j].x, cdec * v[j].y};
              cdec *= am[j];
            }
        }
        for (int m = nch; m < ((nch + 3) & ~3); ++m) coef[b * LS + m] = (f32x2_t){0.f, 0.f};
        beamA[b] = cdec;
      }
    }
    if (nch == 0 && h == 0 && rb == 0) {  // step 1: the first chain rows, and the parents must all be 0
      for (int b = tid; b < nb; b += NT) {
        if (a.parent[(size_t)r * n + b0 + b] != 0) *a.flag = a.epoch;
        int32_t* row = a.chain_out + ((size_t)r * a.B_max + b0 + b) * L;
        row[0] = b0 + b;
        for (int m = 1; m < L; ++m) row[m] = -1;
      }
      if (c.tile == S.ntile - 1)
        for (int idx = tid; idx < (a.B_max - n) * L; idx += NT) a.chain_out[((size_t)r * a.B_max + n) * L + idx] = -1;
    }
    __syncthreads();  // coefficient table ready
    __builtin_amdgcn_s_setprio(1);
    // ---- per 16-beam tile: S_ctx contraction, replay, new record u, output ----
    const int dvl = wave * 16 + 4 * gq;  // this lane's rows within the row block: dvl .. dvl + 3
    const int dv0 = rb * RB + dvl;
    float* u_wr = a.rec_u + arena * d_v;
#pragma unroll
    for (int mt = 0; mt < kTiles; ++mt) {
      if (mt * 16 >= nb) break;
      const int bb = mt * 16 + col;
      const int bc = min(bb, nb - 1);
      floatx4_t pk = (floatx4_t){0.f, 0.f, 0.f, 0.f}, pq = (floatx4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k2 = 0; k2 < kKS; ++k2) {
        const int off = bb * kRow + (((k2 * 4 + gq) ^ ONELA_SWZ(bb)) << 4);
        const bf16x8_t bk = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xk + off));
        const bf16x8_t bq = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xq + off));
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[k2][hl], bk, pk, 0, 0, 0);
          pq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[k2][hl], bq, pq, 0, 0, 0);
        }
      }
      floatx4_t P = (floatx4_t){0.f, 0.f, 0.f, 0.f}, Q = (floatx4_t){0.f, 0.f, 0.f, 0.f};
      if (fast) {
        // the places of eight chain positions in one read, then four records at a time, their coefficient and
        // u reads issued together
        for (int m8 = 0; m8 < nch; m8 += 8) {
          const u32x2_t lw = *reinterpret_cast<const u32x2_t*>(li_t + bc * LIS + m8);
#pragma unroll
          for (int h4 = 0; h4 < 2; ++h4) {
            const int m0 = m8 + 4 * h4;
            if (m0 >= nch) break;
            const unsigned word = h4 ? lw.y : lw.x;
            int d[4];
            f32x2_t cf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // past the chain: record 0, with the zero coefficient written there
              d[j] = m0 + j < nch ? (int)((word >> (8 * j)) & 255u) : 0;
              cf[j] = coef[bc * LS + m0 + j];
            }
            f32x4_t uu[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              uu[j] = *reinterpret_cast<const f32x4_t*>(ud + d[j] * (RB * 4) + (((dvl >> 2) ^ (d[j] & (UP - 1))) << 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                P[e] += cf[j].x * uu[j][e];
                Q[e] += cf[j].y * uu[j][e];
              }
          }
        }
      } else {
        const int32_t* crow = a.chain_out + ((size_t)r * a.B_max + pm_t[bc]) * L;
        for (int m = 0; m < nch; ++m) {
          const f32x2_t cf = coef[bc * LS + m];
          const f32x4_t uu = *reinterpret_cast<const f32x4_t*>(u_rd + (size_t)crow[m] * d_v + dv0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            P[e] += cf.x * uu[e];
            Q[e] += cf.y * uu[e];
          }
        }
      }
      if (bb < nb) {
        const int beam = pm_t[bb];
        const float A = beamA[bb], kq = beamKq[bb];
        const float al = al_t[bb], be = be_t[bb];
        const int vc = dvl >> 3;  // 16-byte piece of the v row block
        const f32x2_t vv = *reinterpret_cast<const f32x2_t*>(xv + bb * RB * 2 + ((vc ^ (bb & (VP - 1))) << 4) + (gq & 1) * 8);
        const uint32_t w0 = __float_as_uint(vv.x), w1 = __float_as_uint(vv.y);
        const float v4[4] = {bf16_bits_to_f32(w0 & 0xFFFFu), bf16_bits_to_f32(w0 >> 16), bf16_bits_to_f32(w1 & 0xFFFFu),
                             bf16_bits_to_f32(w1 >> 16)};
        f32x4_t u4, o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float uu = be * (v4[e] - al * (A * pk[e] + P[e]));
          u4[e] = uu;
          o4[e] = al * (A * pq[e] + Q[e]) + kq * uu;
        }
        const unsigned own = (unsigned)(nch * a.B_max + beam);
        __builtin_amdgcn_s_setprio(2);
        *reinterpret_cast<f32x4_t*>(u_wr + (size_t)own * d_v + dv0) = u4;
        *reinterpret_cast<f32x4_t*>(a.o + (rrow + (size_t)beam * H) * d_v + dv0) = o4;
        __builtin_amdgcn_s_setprio(1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // the next tile overwrites the LDS
  }
}

#undef ONELA_SWZ

// ---------------------------------------------------------------------------------------------------------
bool fused_supported(int d_k, int d_v, int L_max) {
  return (d_k == 128 || d_k == 64 || d_k == 256) && d_v % 32 == 0 && d_v >= 32 && d_v <= 256 && L_max <= 64 &&
         fused_lds_bytes(16, L_max, d_k, d_v) <= 160 * 1024;
}

size_t fused_lds_bytes(int tile, int L_max, int d_k, int d_v) {
  return (size_t)fused_layout(tile, L_max, row_block(d_v), d_k).total;
}

int fused_pick_tile(int d_k, int d_v, int L_max, int requested) {
  if (requested) return requested;
  // 32-beam tiles where two workgroups still fit per CU, or where 16-beam tiles would not fit two either
  return fused_lds_bytes(32, L_max, d_k, d_v) <= 80 * 1024 || fused_lds_bytes(16, L_max, d_k, d_v) > 80 * 1024
             ? 32 : 16;
}

namespace {
// Bytes of the largest plan area of a configuration (either tile size); the processing order follows it.
size_t plan_area_bytes(int R, int B_max, int L_max) {
  size_t most = 0;
  for (int nb : {16, 32}) most = std::max(most, (size_t)R * ((B_max + nb - 1) / nb) * plan_layout(nb, L_max).bytes);
  return (most + 255) & ~(size_t)255;
}
}  // namespace

size_t fused_plan_bytes(int R, int B_max, int L_max) {
  return plan_area_bytes(R, B_max, L_max) + (size_t)R * B_max * 4;  // plans, then rank[R][B_max]
}

namespace {
using FusedKernel = void (*)(StepArgs, const unsigned char*, int, int, int, Sched);
FusedKernel fused_kernel_for(int tile, int rb, int d_k) {
#define ONELA_FUSED_RB(NB, DK)                          \
  switch (rb) {                                         \
    case 32: return &step_fused_kernel<NB, 32, DK>;     \
    case 64: return &step_fused_kernel<NB, 64, DK>;     \
    case 128: return &step_fused_kernel<NB, 128, DK>;   \
    default: return nullptr;                            \
  }
  if (d_k == 128) {
    if (tile == 16) { ONELA_FUSED_RB(16, 128) }
    if (tile == 32) { ONELA_FUSED_RB(32, 128) }
  } else if (d_k == 64) {
    if (tile == 16) { ONELA_FUSED_RB(16, 64) }
    if (tile == 32) { ONELA_FUSED_RB(32, 64) }
  } else if (d_k == 256) {
    if (tile == 16) { ONELA_FUSED_RB(16, 256) }
    if (tile == 32) { ONELA_FUSED_RB(32, 256) }
  }
#undef ONELA_FUSED_RB
  return nullptr;
}
}  // namespace

hipError_t fused_prepare(int tile, int d_k, int d_v, int L_max, int* grid) {
  const int rb = row_block(d_v);
  FusedKernel k = fused_kernel_for(tile, rb, d_k);
  if (!k) return hipErrorInvalidValue;
  const size_t lds = fused_lds_bytes(tile, L_max, d_k, d_v);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const int threads = 64 * (rb / 16);
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), threads, lds)) !=
      hipSuccess)
    return e;
  *grid = std::max(1, cus * std::max(per_cu, 1));
  return hipSuccess;
}

hipError_t launch_step_fused(const StepArgs& a, int tile, void* plan, int grid, hipStream_t s) {
  const int rb = row_block(a.d_v);
  FusedKernel k = fused_kernel_for(tile, rb, a.d_k);
  if (!k) return hipErrorInvalidValue;
  const PlanLayout pl = plan_layout(tile, a.L_max);
  const int ntile = (a.n + tile - 1) / tile;
  unsigned char* pb = static_cast<unsigned char*>(plan);
  int* rank = reinterpret_cast<int*>(pb + plan_area_bytes(a.R, a.B_max, a.L_max));
  if (a.t > 1) {
    if (tile == 16)
      hipLaunchKernelGGL(ancestry_plan_kernel<16>, dim3((unsigned)a.R), dim3(1024), 0, s, a, pb, pl.bytes, pl.perm,
                         pl.li, rank);
    else
      hipLaunchKernelGGL(ancestry_plan_kernel<32>, dim3((unsigned)a.R), dim3(1024), 0, s, a, pb, pl.bytes, pl.perm,
                         pl.li, rank);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const Sched S = make_sched(a.R * a.H, a.d_v / rb, ntile, grid);
  const int g = std::min(grid, S.njobs);
  hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(64 * (rb / 16)), fused_lds_bytes(tile, a.L_max, a.d_k, a.d_v), s, a, pb,
                     pl.bytes, pl.perm, pl.li, S);
  return hipGetLastError();
}

}  // namespace onela
