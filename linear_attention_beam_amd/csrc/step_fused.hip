// Fused projection-replay decode step for gfx950: ancestry update, bf16 MFMA contraction of the shared
// state, record replay and record append in one kernel ("Scientific Impact Assessment: OneLA", §1: a fused
// GPU kernel reuses S_ctx across beams; paper index page, Abstract).
//
// Workgroup = (request, head, tile of NB beams), or a run of consecutive tiles of one (request, head) when
// the register file admits a single workgroup per CU; d_v / 16 waves of 64 lanes (d_k = 128 fixed).
//   Phase 0  everything that needs nothing from the ancestry goes out in the first round trip: parents,
//            alpha and beta; k, q and v rows of the tile (16-byte loads, held in registers and written to
//            LDS only after the chain rows are requested, so that the two round trips overlap); this
//            wave's S_ctx rows.  Wave w owns d_v rows 16w .. 16w+15 of S_ctx, whose bf16 high and low halves stay
//            in registers for the whole tile (each S_ctx element is read once per tile and reused by all
//            NB beams).  Then the ancestry index ("Scientific Impact Assessment: OneLA", §1 item (3)): each
//            beam's chain is its parent's chain from the previous table plus its own slot; the head-0
//            workgroups write the new table.  The decays along a chain (A = prod alpha, c_j = prod of the
//            alphas after record j) are kept per (request, head, beam) next to the index: a beam reads its
//            parent's row (chain entries and A in one round trip, issued by the thread that holds the parent
//            as soon as it arrives, with no barrier before it), and writes its own (c_j alpha_b for the
//            parent's records, 1 for its own record, A alpha_b) for the next step, so no record alpha is
//            gathered.
//   Phase 1  the u of the chain records (this lane's 4-row piece of each of its NB / 16 beams) starts streaming
//            into a register ring; then 16 lanes per (beam, chain record) take the dot products of the chain
//            keys with k and q (a ring of kD1 keys per lane), and k . q, reduced with DPP inside a 16-lane
//            row; append the record key and alpha.
//   Phase 2  the replay: sum_j c_j (K_j.k) U_j and sum_j c_j (K_j.q) U_j for the NB / 16 beams of this
//            lane, records-major over a ring of kRM records (one when NB = 128 or the chain has one record)
//            x NB / 16 tiles.  Then for 16 beams at a time,
//            v_mfma_f32_16x16x32_bf16 computes [P_k | P_q]^T = S_rows [k | q] over d_k, high then low half
//            into one float32 accumulator.  In the accumulator lane l holds beam l % 16 and d_v rows
//            4 (l / 16) .. +3 of the wave's 16 rows, so the replay works per beam on 16-byte pieces (one
//            float4 load of each chain record's u) and u and o leave as float4 stores:
//              p = A P_k + sum_j c_j (K_j.k) U_j,  u = beta (v - alpha p),
//              o = alpha (A P_q + sum_j c_j (K_j.q) U_j) + (k.q) u.
//   Every gather of phases 1 and 2 is an unconditional load in a software pipeline (indices past the end
//   are clamped to a valid record and the values dropped): the compiler's waits on the in-order vmcnt then
//   cover exactly the load consumed, not the loads and stores issued after it.
// Workgroups of one (request, head) are mapped to the same XCD (dispatch is round-robin over the 8 XCDs)
// so their S_ctx reads share one L2.
#include <algorithm>

#include "device_common.h"
#include "launchers.h"

namespace onela {

namespace {
constexpr int kDK = 128;             // d_k of the fused kernel
constexpr int kKS = kDK / 32;        // MFMA k-steps
constexpr int kXRow = 2 * kDK + 16;  // bytes per staged key/query row (padded against bank conflicts)
constexpr int kD1 = 4;               // chain keys in flight per lane (phase 1)
constexpr int kRM = 2;               // chain records per tile in flight per lane (phase 2)
constexpr int kChainChunk = 8;      // chain entries per round trip of the parent-row reads
constexpr int kPersistTiles = 4;     // tiles per workgroup when one workgroup fills a CU

template <int V>
struct IntC {
  static constexpr int value = V;
};
constexpr int kPX = 4;               // 16-byte pieces of the k and q rows per thread held in registers
constexpr int kPV = 2;               // 16-byte pieces of the v rows per thread held in registers

struct FusedLds {
  int xs, slot, alph, coef, item, beamA, beamAl, beamBe, beamKq, vs, vrow, total;
};

// Per-beam tables use an odd row stride so that 16 beams read by one wave fall in distinct LDS banks.
__host__ __device__ inline int table_stride(int L) { return L | 1; }

__host__ __device__ inline FusedLds fused_layout(int NB, int L, int d_v) {
  const int LS = table_stride(L);
  FusedLds l;
  int off = 0;
  l.xs = off;      off += 2 * NB * kXRow;  // k rows, then q rows
  l.slot = off;    off += NB * LS * 4;     // chain slots
  l.alph = off;    off += NB * LS * 4;     // c_j
  l.coef = off;    off += NB * LS * 8;     // (c_j (K_j . k), c_j (K_j . q)) pairs
  l.item = off;    off += NB * L * 8;      // phase-1 work list: (slot, bb << 16 | bb * LS + m)
  l.beamA = off;   off += NB * 4;
  l.beamAl = off;  off += NB * 4;
  l.beamBe = off;  off += NB * 4;
  l.beamKq = off;  off += NB * 4;
  l.vrow = d_v * 2 + 16;
  l.vs = off;      off += NB * l.vrow;     // v rows (bf16, padded like the k and q rows)
  l.total = off;
  return l;
}
// LDS a workgroup may take without LDS cutting the VGPR-limited occupancy (4 waves per SIMD, 16 per CU):
// 160 KB per CU shared by 16 / (d_v / 16) workgroups.
inline size_t lds_budget(int d_v) { return (size_t)640 * d_v; }
}  // namespace

template <int NB, bool PERSIST>
__global__ __launch_bounds__(1024) void step_fused_kernel(StepArgs a, int ntile, int tps) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int L = a.L_max, H = a.H, n = a.n, d_v = a.d_v;
  const int LS = table_stride(L);
  const FusedLds lay = fused_layout(NB, L, d_v);
  const int nthreads = blockDim.x;

  // ---- workgroup -> (request, head, run of tps consecutive tiles); workgroups of one (request, head) share
  // an XCD ----
  const int nsplit = (ntile + tps - 1) / tps;
  int rh, split;
  if (((a.R * H) & 7) == 0) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    rh = (j / nsplit) * 8 + x;
    split = j - (j / nsplit) * nsplit;
  } else {
    rh = blockIdx.x / nsplit;
    split = blockIdx.x - rh * nsplit;
  }
  const int r = rh / H, h = rh - r * H;
  const int nch = a.t - 1;
  const size_t arena = (size_t)rh * a.slots;
  // S_ctx rows of a wave.  Fragment file per (request, head): [hl][w][ks][mi][lane][8], rows
  // 32 w + 16 mi + lane % 16; wave x takes the block w = x / 2, mi = x % 2.  Wave w owns d_v rows
  // 16w .. 16w+15; their bf16 high and low halves stay in registers while the workgroup runs.
  bf16x8_t sf[kKS][2];
  auto load_sf = [&](int wave, int lane) {
    const int W = d_v / 32;
    const size_t half = (size_t)W * kKS * 2 * 64;  // fragments per half
    const u32x4_t* __restrict__ fr = reinterpret_cast<const u32x4_t*>(a.sctx_frag) + (size_t)rh * 2 * half;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        sf[ks][hl] = __builtin_bit_cast(
            bf16x8_t, fr[hl * half + (((size_t)(wave >> 1) * kKS + ks) * 2 + (wave & 1)) * 64 + lane]);
  };

  auto do_tile = [&](const int tile, const int tid) {
    unsigned char* xs = lds + lay.xs;
    unsigned char* vs = lds + lay.vs;
    int* slot_tab = reinterpret_cast<int*>(lds + lay.slot);
    float* c_tab = reinterpret_cast<float*>(lds + lay.alph);
    f32x2_t* coef = reinterpret_cast<f32x2_t*>(lds + lay.coef);
    int2* item_tab = reinterpret_cast<int2*>(lds + lay.item);
    float* beamA = reinterpret_cast<float*>(lds + lay.beamA);
    float* beamAl = reinterpret_cast<float*>(lds + lay.beamAl);
    float* beamBe = reinterpret_cast<float*>(lds + lay.beamBe);
    float* beamKq = reinterpret_cast<float*>(lds + lay.beamKq);
    const int lane = tid & 63, wave = tid >> 6;
    const int b0 = tile * NB;
    const int nb = min(NB, n - b0);
    // Uniform per-workgroup bases; per-lane offsets are 32-bit (the host checks that they fit).
    const size_t row0 = ((size_t)r * n + b0) * H + h;  // input row of beam b0 at this head
    const uint16_t* __restrict__ qin = static_cast<const uint16_t*>(a.q) + row0 * kDK;
    const uint16_t* __restrict__ kin = static_cast<const uint16_t*>(a.k) + row0 * kDK;
    const uint16_t* __restrict__ vin = static_cast<const uint16_t*>(a.v) + row0 * d_v;
    float* __restrict__ o_wr = a.o + row0 * d_v;
    const unsigned hk = (unsigned)H * kDK, hv = (unsigned)H * d_v;  // beam strides of the inputs
    // Records are read only at slots of earlier steps and written only at this step's slots, so the read
    // and write views never touch the same element.
    const uint16_t* __restrict__ k_rd = static_cast<const uint16_t*>(a.rec_k) + arena * kDK;
    uint16_t* __restrict__ k_wr = static_cast<uint16_t*>(a.rec_k) + arena * kDK;
    // u arena of this (request, head); d_v is a multiple of 32 here, so d_v16 = d_v
    const size_t u_arena = (size_t)rh * u_slots16(a.slots) * d_v;
    const float* __restrict__ u_rd = a.rec_u + u_arena;
    float* __restrict__ u_wr = a.rec_u + u_arena;
    float* __restrict__ al_wr = a.rec_alpha + arena;
    auto in_row = [&](int bb) { return row0 + (size_t)bb * H; };

    // ---- phase 0: parents, alpha, beta; k, q and v into LDS; the S_ctx rows into registers.  Every load
    // goes out before the first value is used: thread tid < NB keeps beam tid's parent, alpha and beta in
    // registers until the k, q, v and S_ctx requests have been issued (nthreads = 4 d_v >= NB). ----
    // loads are issued unconditionally (clamped indices, values dropped afterwards) so that the compiler can
    // count them exactly and later waits do not cover loads issued after the one they need
    const int tb = min(tid, nb - 1);
    int pP = a.parent[(size_t)r * n + b0 + tb];
    float pAl = a.alpha[in_row(tb)];
    float pBe = a.beta[in_row(tb)];
    __builtin_amdgcn_sched_barrier(0);  // keep these first in issue order
    // k, q and v of the tile go to registers now and to LDS only after the chain rows are requested, so
    // the chain round trip overlaps this one
    const int vc = d_v >> 3;  // 16-byte pieces per v row
    auto x_piece = [&](int idx) -> u32x4_t {  // idx < NB * 32; rows < NB are keys, the others queries
      const int row = idx >> 4, c = idx & 15;
      const int bb = row < NB ? row : row - NB;
      u32x4_t val = *reinterpret_cast<const u32x4_t*>((row < NB ? kin : qin) + (unsigned)min(bb, nb - 1) * hk + c * 8);
      if (bb >= nb) val = (u32x4_t){0u, 0u, 0u, 0u};
      return val;
    };
    auto v_piece = [&](int idx) -> u32x4_t {  // idx < NB * vc
      const int bb = idx / vc, c = idx - bb * vc;
      u32x4_t val = *reinterpret_cast<const u32x4_t*>(vin + (unsigned)min(bb, nb - 1) * hv + c * 8);
      if (bb >= nb) val = (u32x4_t){0u, 0u, 0u, 0u};
      return val;
    };
    u32x4_t XR[kPX], VR[kPV];
#pragma unroll
    for (int u = 0; u < kPX; ++u) XR[u] = x_piece(min(tid + u * nthreads, NB * 32 - 1));
#pragma unroll
    for (int u = 0; u < kPV; ++u) VR[u] = v_piece(min(tid + u * nthreads, NB * vc - 1));
    auto store_x = [&]() {
#pragma unroll
      for (int u = 0; u < kPX; ++u) {
        const int idx = tid + u * nthreads;
        if (idx < NB * 32) *reinterpret_cast<u32x4_t*>(xs + (idx >> 4) * kXRow + (idx & 15) * 16) = XR[u];
      }
      for (int idx = tid + kPX * nthreads; idx < NB * 32; idx += nthreads)
        *reinterpret_cast<u32x4_t*>(xs + (idx >> 4) * kXRow + (idx & 15) * 16) = x_piece(idx);
#pragma unroll
      for (int u = 0; u < kPV; ++u) {
        const int idx = tid + u * nthreads;
        if (idx < NB * vc) {
          const int bb = idx / vc;
          *reinterpret_cast<u32x4_t*>(vs + bb * lay.vrow + (idx - bb * vc) * 16) = VR[u];
        }
      }
      for (int idx = tid + kPV * nthreads; idx < NB * vc; idx += nthreads) {
        const int bb = idx / vc;
        *reinterpret_cast<u32x4_t*>(vs + bb * lay.vrow + (idx - bb * vc) * 16) = v_piece(idx);
      }
    };
    const int gq = lane >> 4, col = lane & 15;
    const int dv0 = wave * 16 + 4 * gq;  // this lane's d_v rows: dv0 .. dv0+3
    constexpr int kTiles = NB / 16;
    if constexpr (!PERSIST) load_sf(wave, lane);
    __builtin_amdgcn_sched_barrier(0);  // every streaming request is out before the parents are consumed
    if (tid >= nb) {
      pP = 0;
      pAl = 0.f;
      pBe = 0.f;
    }
    // ---- phase 0 (cont.): thread tid < NB holds beam tid's parent and reads the parent's chain row and decay
    // row itself, as soon as the parent has arrived (no barrier before this round trip); this step's rows.
    // Loads are unconditional (entries past the chain are clamped to its last one and dropped). ----
    const int drow = L + 1;  // decay row: c_0 .. c_{L-1}, then A
    if (tid < NB) {
      // sticky flag; decode as a child of beam 0 so that accesses stay in bounds
      if (tid < nb && (pP < 0 || pP >= a.b_prev)) {
        *a.flag = a.epoch;
        pP = 0;
      }
      beamAl[tid] = pAl;
      beamBe[tid] = pBe;
      const bool live = tid < nb;
      float* dout = a.decay_out + ((size_t)rh * a.B_max + b0 + tid) * drow;
      int32_t* cout = a.chain_out + ((size_t)r * a.B_max + b0 + tid) * L;
      if (nch > 0) {
        const int32_t* crow = a.chain_prev + ((size_t)r * a.B_max + pP) * L;
        const float* drw = a.decay_prev + ((size_t)rh * a.B_max + pP) * drow;
        const float Ap = drw[L];
        for (int m0 = 0; m0 < nch; m0 += kChainChunk) {
          int raw[kChainChunk];
          float dec[kChainChunk];
#pragma unroll
          for (int u = 0; u < kChainChunk; ++u) {
            const int m = min(m0 + u, nch - 1);
            raw[u] = crow[m];
            dec[u] = drw[m];
          }
#pragma unroll
          for (int u = 0; u < kChainChunk; ++u) {
            const int m = m0 + u;
            if (live && m < nch) {
              const int sl = raw[u] < 0 ? 0 : (raw[u] >= a.slots ? a.slots - 1 : raw[u]);
              slot_tab[tid * LS + m] = sl;
              c_tab[tid * LS + m] = dec[u];
              item_tab[tid * nch + m] = make_int2(sl, (tid << 16) | (tid * LS + m));
              dout[m] = dec[u] * pAl;
              if (h == 0) cout[m] = raw[u];
            }
          }
        }
        if (live) {
          dout[nch] = 1.f;
          dout[L] = Ap * pAl;
        }
        beamA[tid] = live ? Ap : 0.f;
      } else {
        if (live) {
          dout[0] = 1.f;
          dout[L] = pAl;
        }
        beamA[tid] = live ? 1.f : 0.f;
      }
      if (h == 0 && live) {  // the rest of the row: own slot, then -1
        for (int m = nch; m < L; ++m) cout[m] = m == nch ? nch * a.B_max + b0 + tid : -1;
      }
    }
    if (h == 0 && tile == ntile - 1) {  // rows of beams >= n are all -1
      for (int idx = tid; idx < (a.B_max - n) * L; idx += nthreads)
        a.chain_out[((size_t)r * a.B_max + n) * L + idx] = -1;
    }
    store_x();
    __syncthreads();

    // ---- after the chain tables: every remaining global load is a gather whose address comes from LDS.  The
    // gathers run as software pipelines of unconditional loads (indices past the end are clamped to a valid
    // record and their values dropped), so that the compiler's in-order vmcnt waits cover exactly the load
    // being consumed and never the ones issued after it.
    const int g16 = tid >> 4, j16 = tid & 15;
    const int ngroups = nthreads >> 4;
    auto rest = [&](auto rm_c) {
      constexpr int RM = decltype(rm_c)::value;  // chain records per tile in flight in the u ring (0: no chain)
      constexpr int NU = RM > 0 ? RM * kTiles : 1;
      int bcs[kTiles];  // this lane's beam in each 16-beam tile, clamped to the tile's last beam
#pragma unroll
      for (int mt = 0; mt < kTiles; ++mt) bcs[mt] = min(mt * 16 + col, nb - 1);
      auto u_load = [&](int mt, int m) -> f32x4_t {
        const unsigned uo = u_index((unsigned)slot_tab[bcs[mt] * LS + m], (unsigned)dv0, (unsigned)d_v);
        return *reinterpret_cast<const f32x4_t*>(u_rd + uo);
      };
      // u ring, records-major: U[r * kTiles + mt] holds record m0 + r of tile mt.  Its first RM records go out
      // now and land during phase 1.
      f32x4_t U[NU];
      if constexpr (RM > 0) {
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int mt = 0; mt < kTiles; ++mt) U[r * kTiles + mt] = u_load(mt, min(r, nch - 1));
      }

      // ---- phase 1: 16 lanes per (beam, chain record): K_j . k and K_j . q into the coefficient table.  Group g
      // takes items g, g + ngroups, ...; a ring of kD1 chain keys per lane. ----
      if constexpr (RM > 0) {
        const int items = nb * nch;
        const int kmax = (items + ngroups - 1) / ngroups;
        u32x4_t K[kD1];
        int IY[kD1];
        auto k_load = [&](int kk, int d) {
          const int2 e = item_tab[min(kk * ngroups + g16, items - 1)];
          IY[d] = e.y;
          K[d] = *reinterpret_cast<const u32x4_t*>(k_rd + ((unsigned)e.x * kDK + j16 * 8));
        };
        auto k_use = [&](int kk, int d) {
          if (kk * ngroups + g16 < items) {  // uniform over the 16 lanes of the group
            const int pos = IY[d] & 0xFFFF, bb = IY[d] >> 16;
            const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(xs + bb * kXRow + j16 * 16);
            const u32x4_t qx = *reinterpret_cast<const u32x4_t*>(xs + (NB + bb) * kXRow + j16 * 16);
            const float dk = row16_sum(dot8_bf16(K[d], kx));
            const float dq = row16_sum(dot8_bf16(K[d], qx));
            if (j16 == 0) {
              const float c = c_tab[pos];
              coef[pos] = (f32x2_t){c * dk, c * dq};
            }
          }
        };
#pragma unroll
        for (int d = 0; d < kD1; ++d) k_load(d, d);
        int k0 = 0;
        for (; k0 + kD1 < kmax; k0 += kD1) {
#pragma unroll
          for (int d = 0; d < kD1; ++d) {
            k_use(k0 + d, d);
            k_load(k0 + kD1 + d, d);
          }
        }
#pragma unroll
        for (int d = 0; d < kD1; ++d) k_use(k0 + d, d);
      }
      // k . q of every beam; append the record key and alpha
      for (int bb = g16; bb < nb; bb += ngroups) {
        const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(xs + bb * kXRow + j16 * 16);
        const u32x4_t qx = *reinterpret_cast<const u32x4_t*>(xs + (NB + bb) * kXRow + j16 * 16);
        const float kq = row16_sum(dot8_bf16(kx, qx));
        const unsigned own = (unsigned)(nch * a.B_max + b0 + bb);
        *reinterpret_cast<u32x4_t*>(k_wr + (own * kDK + j16 * 8)) = kx;
        if (j16 == 0) {
          beamKq[bb] = kq;
          al_wr[own] = beamAl[bb];
        }
      }
      __syncthreads();

      // ---- phase 2: the replay over the u ring (sums per tile in P, Q), then per tile the MFMA contraction,
      // u and o ----
      floatx4_t P[kTiles], Q[kTiles];
#pragma unroll
      for (int mt = 0; mt < kTiles; ++mt) {
        P[mt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
        Q[mt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
      }
      if constexpr (RM > 0) {
        auto acc = [&](int mt, int m, int i) {
          if (mt * 16 < nb) {
            const f32x2_t c = coef[bcs[mt] * LS + m];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              P[mt][e] += c.x * U[i][e];
              Q[mt][e] += c.y * U[i][e];
            }
          }
        };
        int m0 = 0;
        for (; m0 + RM < nch; m0 += RM) {
#pragma unroll
          for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int mt = 0; mt < kTiles; ++mt) {
              acc(mt, m0 + r, r * kTiles + mt);
              U[r * kTiles + mt] = u_load(mt, min(m0 + RM + r, nch - 1));
            }
        }
#pragma unroll
        for (int r = 0; r < RM; ++r)
          if (m0 + r < nch) {
#pragma unroll
            for (int mt = 0; mt < kTiles; ++mt) acc(mt, m0 + r, r * kTiles + mt);
          }
      }
#pragma unroll
      for (int mt = 0; mt < kTiles; ++mt) {
        if (mt * 16 >= nb) break;
        const int bb = mt * 16 + col;
        floatx4_t pk = (floatx4_t){0.f, 0.f, 0.f, 0.f}, pq = (floatx4_t){0.f, 0.f, 0.f, 0.f};
        // B operand: lane l holds column (beam) l % 16, k = 8 (l / 16) .. +7 of this k-step
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          const bf16x8_t bk = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + bb * kXRow + ks * 64 + gq * 16));
          const bf16x8_t bq = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + (NB + bb) * kXRow + ks * 64 + gq * 16));
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[ks][hl], bk, pk, 0, 0, 0);
            pq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[ks][hl], bq, pq, 0, 0, 0);
          }
        }
        if (bb < nb) {
          const float A = beamA[bb], al = beamAl[bb], be = beamBe[bb], kq = beamKq[bb];
          const unsigned own = (unsigned)(nch * a.B_max + b0 + bb);
          const f32x2_t vv = *reinterpret_cast<const f32x2_t*>(vs + bb * lay.vrow + dv0 * 2);
          const uint32_t w0 = __float_as_uint(vv.x), w1 = __float_as_uint(vv.y);
          const float v4[4] = {bf16_bits_to_f32(w0 & 0xFFFFu), bf16_bits_to_f32(w0 >> 16),
                               bf16_bits_to_f32(w1 & 0xFFFFu), bf16_bits_to_f32(w1 >> 16)};
          f32x4_t u4, o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float uu = be * (v4[e] - al * (A * pk[e] + P[mt][e]));
            u4[e] = uu;
            o4[e] = al * (A * pq[e] + Q[mt][e]) + kq * uu;
          }
          *reinterpret_cast<f32x4_t*>(u_wr + u_index(own, (unsigned)dv0, (unsigned)d_v)) = u4;  // 1 KB per wave
          *reinterpret_cast<f32x4_t*>(o_wr + ((unsigned)bb * hv + dv0)) = o4;
        }
      }
    };
    if (nch == 0)
      rest(IntC<0>{});
    else if (nch == 1)
      rest(IntC<1>{});
    else
      rest(IntC<(NB >= 128 ? 1 : kRM)>{});  // 8 tiles per lane: one record per tile in flight
  };

  if constexpr (PERSIST) {
    load_sf((int)threadIdx.x >> 6, (int)threadIdx.x & 63);
    const int tile_end = min(ntile, (split + 1) * tps);
    for (int tile = split * tps; tile < tile_end; ++tile) {
      // the thread index is laundered per tile, so that the compiler derives the per-lane addresses next to
      // their use instead of keeping them live (and spilled) across the loop
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      do_tile(tile, tid);
      if (tile + 1 < tile_end) __syncthreads();  // the next tile overwrites the LDS tables
    }
  } else {
    do_tile(split, (int)threadIdx.x);
  }
}

bool fused_supported(int d_k, int d_v, int L_max) {
  return d_k == kDK && d_v % 32 == 0 && d_v >= 32 && d_v <= 256 && fused_lds_bytes(16, L_max, d_v) <= 160 * 1024;
}

size_t fused_lds_bytes(int tile, int L_max, int d_v) {
  return (size_t)fused_layout(tile, L_max, d_v).total;
}

int fused_pick_tile(int R, int H, int n, int d_v, int L_max, int requested) {
  if (requested) return requested;
  const long G = (long)R * H;
  const int cands[3] = {64, 32, 16};
  for (int c : cands) {
    const long wgs = G * ((n + c - 1) / c);
    if (wgs >= 1024 && fused_lds_bytes(c, L_max, d_v) <= lds_budget(d_v)) return c;
  }
  return 16;
}

namespace {
using FusedKernel = void (*)(StepArgs, int, int);
hipError_t launch_fused_as(FusedKernel k, dim3 grid, dim3 block, size_t lds, hipStream_t s, const StepArgs& a,
                           int ntile, int tps) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, grid, block, lds, s, a, ntile, tps);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_step_fused(const StepArgs& a, int tile, hipStream_t s) {
  const int ntile = (a.n + tile - 1) / tile;
  // A workgroup has d_v / 16 waves of up to 128 VGPRs: the register file admits 16 / (d_v / 16) per CU.  When
  // it admits one, each workgroup runs kPersistTiles consecutive tiles of its (request, head): no CU then idles
  // between one workgroup's last store and the next one's launch, and S_ctx is read once per run.
  const bool persist = 16 / (a.d_v / 16) < 2;
  const int tps = persist ? std::min(ntile, kPersistTiles) : 1;
  const int nsplit = (ntile + tps - 1) / tps;
  dim3 grid((unsigned)((size_t)a.R * a.H * nsplit)), block(4 * a.d_v);
  const size_t lds = fused_lds_bytes(tile, a.L_max, a.d_v);
#define ONELA_FUSED_CASE(NB)                                                                     \
  case NB:                                                                                       \
    return persist ? launch_fused_as(&step_fused_kernel<NB, true>, grid, block, lds, s, a, ntile, tps) \
                   : launch_fused_as(&step_fused_kernel<NB, false>, grid, block, lds, s, a, ntile, tps);
  switch (tile) {
    ONELA_FUSED_CASE(16)
    ONELA_FUSED_CASE(32)
    ONELA_FUSED_CASE(64)
    ONELA_FUSED_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef ONELA_FUSED_CASE
}

}  // namespace onela
