// Beam selection for gfx950: the top n_beams of all (parent, candidate) scores of each request, best first,
// which become the next decode step's parents ("Scientific Impact Assessment: OneLA", §1 Core Contribution:
// beams are pruned, reordered and fanned out, each survivor naming its parent).
//
// Rule: candidate (b, c) scores s = beam_score[b] + logp[b, c] (one float32 addition); higher score ranks
// first, and equal scores rank by the smaller flat index f = b * n_cand + c.  Each candidate becomes one
// 64-bit key whose unsigned order is exactly that ranking: the high word maps the float32 score to an
// order-preserving unsigned integer (-0 and +0 map alike), the low word is ~f.  Keys are unique, so the
// top set and its order are unique too.
//
// Selection without sorting everything: a workgroup holds up to 8192 keys in registers (1024 threads x 8; the
// chunk pass takes 512 x 16 when there are at least two chunks per CU) and an MSB-first radix select finds
// the smallest key T such that exactly K keys are >= T (8-bit digits from the highest bit where the keys
// differ, one LDS histogram per pass; it stops as soon as a whole digit bucket is taken, or once the bucket
// holding T has at most 64 keys, one wavefront picks T from them).  The keys >= T are then compacted.
//   Chunk   each workgroup reduces 8192 keys of one request to its K best (unordered); repeated until a
//           request has at most 8192 keys left (one launch for 32 x 512 x 256 -> 512).
//   Finish  one workgroup selects a request's K keys from at most 8192 (chunk survivors or the scores
//           themselves), orders them (sorted runs of 64, then ranks by binary search) and writes parent,
//           token, score.
// The two phases are separate launches: a single launch whose last-arriving chunk workgroup finishes the
// request needs a device-scope release per workgroup, and on this chip each one writes back the XCD's L2;
// measured, that costs more than the launch boundary it saves.  Key 0 pads short chunks and ranks below
// every real key.
#include <mutex>

#include "device_common.h"
#include "launchers.h"

// Whole-wave 64-bit unsigned min / max of the device library (the HIP headers declare them only under an
// opt-in macro).
extern "C" __device__ __attribute__((const)) unsigned long long __ockl_wfred_min_u64(unsigned long long);
extern "C" __device__ __attribute__((const)) unsigned long long __ockl_wfred_max_u64(unsigned long long);

namespace onela {

namespace {
constexpr int kThreads = 1024;                 // finish workgroup: threads, keys per thread
constexpr int kPerThread = 8;
constexpr int kChunk = kThreads * kPerThread;  // keys per workgroup
constexpr int kMaxBeams = 2048;
constexpr int kHistCopies = 8;                 // lanes l with l % 8 == c share histogram copy c
constexpr int kHistStride = 260;               // ints per copy: the copies of one digit sit in different banks
constexpr int kBucket = 64;                    // a threshold bucket this small is finished by one wavefront

__device__ __forceinline__ uint32_t score_order(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t f) {
  return ((uint64_t)score_order(s) << 32) | (uint64_t)(~f);
}

// The score a key was made from: score_order is one-to-one on every float but the two zeros, which it maps
// alike (a zero comes back as +0).
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// LDS of one selection workgroup: the radix histograms and choices, per-wave extremes, and (finish only) the
// K survivors and their sorted runs of 64.
struct alignas(16) SelLds {
  int hist[kHistCopies][kHistStride];
  unsigned long long wmin[kThreads / 64], wmax[kThreads / 64];
  uint64_t bucket[kBucket], thr;
  int digit, rank, count, n_out, n_bucket;
  uint64_t best[kMaxBeams];
  uint64_t sorted[kMaxBeams];
};

// This thread's keys of positions [base, base + T P) of request r, position base + e T + tid in slot e,
// padded with 0 past n_in (T threads, P keys each).  Built from the scores (src == nullptr) or read from a key
// buffer.
template <int T, int P>
__device__ __forceinline__ void load_keys(uint64_t (&key)[P], const float* beam_scores,
                                          const float* logp, const uint64_t* src, long n_in, int n_prev,
                                          int n_cand, int r, long base) {
  const int tid = threadIdx.x;
  if (src == nullptr) {
    const float* bs = beam_scores + (size_t)r * n_prev;
    const float* lp = logp + (size_t)r * n_in;
    // slot e's flat index is f0 + e T: its beam f / n_cand is stepped (quotient and remainder of T added, one
    // carry) rather than divided per slot, so the beam-score loads do not wait on P divisions
    const uint32_t nc = (uint32_t)n_cand, f0 = (uint32_t)(base + tid);
    const uint32_t dq = (uint32_t)T / nc, dr = (uint32_t)T - dq * nc;
    uint32_t q = f0 / nc, rm = f0 - q * nc;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const long i = base + e * T + tid;
      uint64_t k = 0;
      if (i < n_in) {
        const uint32_t f = (uint32_t)i;
        k = make_key(bs[q] + lp[f], f);
      }
      key[e] = k;
      q += dq;
      rm += dr;
      if (rm >= nc) {
        rm -= nc;
        ++q;
      }
    }
  } else {
    const uint64_t* s = src + (size_t)r * n_in;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const long i = base + e * T + tid;
      key[e] = i < n_in ? s[i] : 0ull;
    }
  }
}

// The value of lane (lane ^ off).  Within a row of 16 lanes (off = 1, 2, 4, 8) by DPP register moves: quad
// permutations for 1 and 2; for 4 and 8 a row shift each way (row_shl:n gives lane i the value of lane i + n,
// row_shr:n that of lane i - n), and the lane takes the one that stays in its row.  Across rows (16, 32) by a
// permute through the LDS crossbar.  off must be a constant after inlining.
__device__ __forceinline__ uint32_t xor_lane32(uint32_t v, int off, int lane) {
  const int x = (int)v;
  if (off == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  if (off == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  if (off == 4) {
    const int up = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, false);  // row_shl:4
    const int dn = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, false);  // row_shr:4
    return (uint32_t)((lane & 4) ? dn : up);
  }
  if (off == 8) {
    const int up = __builtin_amdgcn_mov_dpp(x, 0x108, 0xF, 0xF, false);  // row_shl:8
    const int dn = __builtin_amdgcn_mov_dpp(x, 0x118, 0xF, 0xF, false);  // row_shr:8
    return (uint32_t)((lane & 8) ? dn : up);
  }
  return (uint32_t)__shfl_xor(x, off, 64);
}
__device__ __forceinline__ unsigned long long xor_lane64(unsigned long long v, int off, int lane) {
  return ((unsigned long long)xor_lane32((uint32_t)(v >> 32), off, lane) << 32) | xor_lane32((uint32_t)v, off, lane);
}

// The rank-th largest of the cnt (<= kBucket) keys k with (k & mask) == prefix: they are gathered in LDS, and
// each lane of one wavefront counts the gathered keys above its own.  Every thread must call it.
template <int P>
__device__ __forceinline__ uint64_t bucket_pick(const uint64_t (&key)[P], uint64_t prefix, uint64_t mask,
                                                int cnt, int rank, SelLds& sh) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const bool in = (key[e] & mask) == prefix;  // the keys the last histogram pass counted in the bucket
    const uint64_t take = __ballot(in);
    if (take) {  // one atomic per wavefront
      const int first = __ffsll((long long)take) - 1;
      int base = 0;
      if (lane == first) base = atomicAdd(&sh.n_bucket, __popcll(take));
      base = __shfl(base, first, 64);
      if (in) sh.bucket[base + __popcll(take & ((1ull << lane) - 1))] = key[e];
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const uint64_t x = lane < cnt ? sh.bucket[lane] : 0ull;
    int above = 0;
    for (int j = 0; j < cnt; ++j) above += sh.bucket[j] > x;
    if (lane < cnt && above == rank - 1) sh.thr = x;  // keys are unique: exactly one lane
  }
  __syncthreads();
  return sh.thr;
}

// Smallest key T such that exactly K of the workgroup's unique keys are >= T (requires 1 <= K <= the number
// of nonzero keys).  Every thread must call it.  Digits start at the highest bit where the smallest and the
// largest real key differ: the bits above are common to all of them and would only cost passes that split
// nothing.  Once the bucket that holds T has at most kBucket keys, T is picked from them directly: at
// 32 x 512 x 256 candidates every chunk then needs at most two histogram passes (up to seven before).
template <int T, int P>
__device__ __forceinline__ uint64_t radix_threshold(const uint64_t (&key)[P], int K, SelLds& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, copy = lane & (kHistCopies - 1);
  unsigned long long lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const unsigned long long k = key[e];
    if (k != 0ull) {
      lo = k < lo ? k : lo;
      hi = k > hi ? k : hi;
    }
  }
  lo = __ockl_wfred_min_u64(lo);
  hi = __ockl_wfred_max_u64(hi);
  if (lane == 0) {
    sh.wmin[wave] = lo;
    sh.wmax[wave] = hi;
  }
  for (int i = tid; i < kHistCopies * kHistStride; i += T) (&sh.hist[0][0])[i] = 0;
  if (tid == 0) sh.n_bucket = 0;
  __syncthreads();
  lo = ~0ull;
  hi = 0ull;
#pragma unroll
  for (int w = 0; w < T / 64; ++w) {
    lo = sh.wmin[w] < lo ? sh.wmin[w] : lo;
    hi = sh.wmax[w] > hi ? sh.wmax[w] : hi;
  }
  const uint64_t kmax = hi, diff = hi ^ lo;
  if (diff == 0) return kmax;  // a single real key
  int top = 63 - __clzll((long long)diff);
  uint64_t mask = top == 63 ? 0ull : ~((2ull << top) - 1), prefix = kmax & mask;
  int rank = K;
  for (;;) {
    const int w = top >= 7 ? 8 : top + 1, shift = top - w + 1;
#pragma unroll
    for (int e = 0; e < P; ++e)
      if ((key[e] & mask) == prefix) atomicAdd(&sh.hist[copy][(int)((key[e] >> shift) & 0xFFu)], 1);
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255 - 4l .. 252 - 4l (c[e]: digit 255 - 4l - e): lane order is descending digit
      // order.  The copies are summed and cleared for the next pass.
      int c[4] = {0, 0, 0, 0};
#pragma unroll 2
      for (int x = 0; x < kHistCopies; ++x) {
        int4* h4 = reinterpret_cast<int4*>(&sh.hist[x][252 - 4 * tid]);
        const int4 v = *h4;
        *h4 = make_int4(0, 0, 0, 0);
        c[0] += v.w;
        c[1] += v.z;
        c[2] += v.y;
        c[3] += v.x;
      }
      const int local = c[0] + c[1] + c[2] + c[3];
      int incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (tid >= off) incl += v;
      }
      int run = incl - local;
      if (run < rank && incl >= rank) {  // exactly one lane
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (run + c[e] >= rank) {
            sh.digit = 255 - 4 * tid - e;
            sh.rank = rank - run;
            sh.count = c[e];
            break;
          }
          run += c[e];
        }
      }
    }
    __syncthreads();
    // the next pass's histogram atomics come after this read, and the choice is rewritten only after the
    // next pass's barrier: no barrier is needed here
    const int d = sh.digit, cnt = sh.count;
    rank = sh.rank;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)((1u << w) - 1u) << shift;
    if (cnt == rank || shift == 0) break;  // the whole bucket is taken: exactly K keys are >= prefix
    if (cnt <= kBucket) return bucket_pick(key, prefix, mask, cnt, rank, sh);
    top = shift - 1;
  }
  return prefix;
}

// Write this workgroup's keys >= thr (K of them) to out[0 .. K) in arbitrary order (out: global or LDS).
template <int P>
__device__ __forceinline__ void compact(const uint64_t (&key)[P], uint64_t thr, uint64_t* out, SelLds& sh) {
  if (threadIdx.x == 0) sh.n_out = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const bool mine = key[e] >= thr;
    const uint64_t take = __ballot(mine);
    if (take) {  // one atomic per wave; lanes take consecutive places in lane order
      const int first = __ffsll((long long)take) - 1;
      int base = 0;
      if (lane == first) base = atomicAdd(&sh.n_out, __popcll(take));
      base = __shfl(base, first, 64);
      if (mine) out[base + __popcll(take & ((1ull << lane) - 1))] = key[e];
    }
  }
  __syncthreads();
}

// One chunk of request r: its K best keys (unordered; all keys, 0-padded, when the chunk holds at most K)
// to dst[0 .. K).
template <int T, int P>
__device__ __forceinline__ void reduce_chunk(const float* beam_scores, const float* logp, const uint64_t* src, long n_in,
                             int n_prev, int n_cand, int r, int c, int K, uint64_t* dst, SelLds& sh) {
  uint64_t key[P];
  const long base = (long)c * (T * P);
  load_keys<T, P>(key, beam_scores, logp, src, n_in, n_prev, n_cand, r, base);
  if (n_in - base <= K) {
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int i = e * T + threadIdx.x;
      if (i < K) dst[i] = key[e];
    }
    return;
  }
  compact<P>(key, radix_threshold<T, P>(key, K, sh), dst, sh);
}

// Request r's top K of its n_in (<= kChunk) keys, best first, to parent / token / score.
__device__ __forceinline__ void finish_request(const float* beam_scores, const float* logp, const uint64_t* src, long n_in,
                               int n_prev, int n_cand, int r, int K, int32_t* parent, int32_t* token,
                               float* score, SelLds& sh) {
  uint64_t key[kPerThread];
  load_keys<kThreads, kPerThread>(key, beam_scores, logp, src, n_in, n_prev, n_cand, r, 0);
  compact<kPerThread>(key, radix_threshold<kThreads, kPerThread>(key, K, sh), sh.best, sh);
  // order: each wave sorts runs of 64 survivors in registers (a bitonic network over the lanes, largest
  // first; slots past K hold key 0, which sorts last); then the rank of a survivor is its place in its own
  // run plus, for every other run, the number of that run's keys above it (a binary search).  Keys are
  // unique, so the ranks are a permutation of 0 .. K-1.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nrun = (K + 63) >> 6;
  uint64_t* runs = sh.sorted;
  for (int run = wave; run < nrun; run += kThreads / 64) {
    uint64_t x = run * 64 + lane < K ? sh.best[run * 64 + lane] : 0ull;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1) {
        const uint64_t y = xor_lane64(x, j, lane);
        const bool take_max = ((lane & j) == 0) == ((lane & k) == 0);
        x = take_max ? (x > y ? x : y) : (x < y ? x : y);
      }
    }
    runs[run * 64 + lane] = x;
  }
  __syncthreads();
  // Each survivor's rank is the sum of two halves, each counted by its own thread: its place in its own run plus
  // the searches of the first half of the runs, and the searches of the second half.  The halves go to the
  // histogram space when they fit, else to the survivors' space (read back before the survivors are placed).
  const int half = (nrun + 1) >> 1, nsurv = nrun * 64;
  const bool in_hist = 2 * nsurv <= kHistCopies * kHistStride;
  int* part = in_hist ? &sh.hist[0][0] : reinterpret_cast<int*>(sh.best);
  for (int it = threadIdx.x; it < 2 * nsurv; it += kThreads) {
    const int h = it >= nsurv, i = it - h * nsurv;
    const uint64_t x = runs[i];
    const int own = i >> 6, bl = h * half, bh = min(nrun, bl + half);
    int rank = h ? 0 : (i & 63);
    for (int b0 = bl; b0 < bh; b0 += 8) {  // 8 independent searches in flight
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = b0 + u;
        if (b < bh && b != own) {
          const uint64_t* rb = runs + b * 64;
          int pos = 0;
#pragma unroll
          for (int step = 32; step > 0; step >>= 1)
            if (rb[pos + step - 1] > x) pos += step;
          if (pos == 63 && rb[63] > x) pos = 64;
          rank += pos;
        }
      }
    }
    part[it] = rank;
  }
  __syncthreads();
  if (in_hist) {
    for (int i = threadIdx.x; i < nsurv; i += kThreads) {
      const uint64_t x = runs[i];
      if (x != 0ull) sh.best[part[i] + part[nsurv + i]] = x;  // key 0 is padding
    }
  } else {
    int rk[kMaxBeams / kThreads];
#pragma unroll
    for (int e = 0; e < kMaxBeams / kThreads; ++e) {
      const int i = e * kThreads + threadIdx.x;
      rk[e] = i < nsurv ? part[i] + part[nsurv + i] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kMaxBeams / kThreads; ++e) {
      const int i = e * kThreads + threadIdx.x;
      if (i < nsurv && runs[i] != 0ull) sh.best[rk[e]] = runs[i];
    }
  }
  __syncthreads();
  // the score comes back from the key; a zero score is recomputed from its inputs (the same float32 addition)
  // so that its sign survives
  const float* bs = beam_scores + (size_t)r * n_prev;
  const float* lp = logp + (size_t)r * n_prev * n_cand;
  for (int i = threadIdx.x; i < K; i += kThreads) {
    const uint64_t key = sh.best[i];
    const uint32_t f = ~(uint32_t)key;
    const uint32_t p = f / (uint32_t)n_cand;
    const size_t o = (size_t)r * K + i;
    parent[o] = (int32_t)p;
    token[o] = (int32_t)(f - p * (uint32_t)n_cand);
    const float sc = key_score(key);
    score[o] = sc == 0.f ? bs[p] + lp[f] : sc;
  }
}

// T threads of kChunk / T keys each; two workgroups per CU
template <int T>
__global__ __launch_bounds__(T, T / 128) void select_chunk_kernel(const float* __restrict__ beam_scores,
                                                                const float* __restrict__ logp,
                                                                const uint64_t* __restrict__ src, long n_in,
                                                                int n_prev, int n_cand, int nchunk, int K,
                                                                uint64_t* __restrict__ out) {
  __shared__ SelLds sh;
  const int r = blockIdx.x / nchunk, c = blockIdx.x - r * nchunk;
  reduce_chunk<T, kChunk / T>(beam_scores, logp, src, n_in, n_prev, n_cand, r, c, K, out + ((size_t)r * nchunk + c) * K,
                              sh);
}

__global__ __launch_bounds__(kThreads, 8) void select_finish_kernel(const float* __restrict__ beam_scores,
                                                                 const float* __restrict__ logp,
                                                                 const uint64_t* __restrict__ src, long n_in,
                                                                 int n_prev, int n_cand, int K,
                                                                 int32_t* parent, int32_t* token, float* score) {
  __shared__ SelLds sh;
  finish_request(beam_scores, logp, src, n_in, n_prev, n_cand, blockIdx.x, K, parent, token, score, sh);
}

}  // namespace

// Library-held scratch of the allocation-free entry point, one copy per GPU (zero-initialised at load).
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

int beam_select_max_beams() { return kMaxBeams; }

size_t beam_select_scratch_bytes(int R, long n, int n_beams) {
  // keys surviving the first chunk pass, twice (later passes alternate between the two halves)
  if (n <= kChunk) return 0;
  const long nchunk = (n + kChunk - 1) / kChunk;
  return (size_t)2 * R * nchunk * n_beams * sizeof(uint64_t);
}

size_t beam_select_static_max() { return kStaticScratchBytes; }

hipError_t beam_select_static_scratch(void** ptr) {
  // the array's address on each GPU, looked up once per device with that device current; host code uses
  // this address only (the array's own name is a host-side stand-in)
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {
// Compute units of the current device, looked up once per device.
hipError_t compute_units(int* cus) {
  static std::mutex mu;
  static int count[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!count[dev]) {
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    count[dev] = c > 0 ? c : 1;
  }
  *cus = count[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_beam_select(const float* beam_scores, const float* logp, int R, int n_prev, int n_cand,
                              int n_beams, int32_t* parent, int32_t* token, float* score, void* scratch_buf,
                              hipStream_t s) {
  long n = (long)n_prev * n_cand;
  const int K = n_beams;  // K <= kChunk / 4: every chunk pass at least quarters the keys
  if (n <= kChunk) {
    hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)R), dim3(kThreads), 0, s, beam_scores, logp, nullptr,
                       n, n_prev, n_cand, K, parent, token, score);
    return hipGetLastError();
  }
  const long nchunk0 = (n + kChunk - 1) / kChunk;
  int cus = 0;
  {
    const hipError_t e = compute_units(&cus);
    if (e != hipSuccess) return e;
  }
  uint64_t* buf[2] = {static_cast<uint64_t*>(scratch_buf), static_cast<uint64_t*>(scratch_buf) + (size_t)R * nchunk0 * K};
  const uint64_t* in = nullptr;
  int which = 0;
  while (n > kChunk) {
    const int nchunk = (int)((n + kChunk - 1) / kChunk);
    // With two chunks per CU or more, 512-thread workgroups (half the waves to dispatch, cheaper barriers);
    // with fewer, 1024 threads hide more latency per CU.  At 32 x 512 x 256: 25.7 against 26.8 us per call;
    // at 16 x 512 x 256 (one chunk per CU) 23.1 against 21.7.
    const unsigned nwg = (unsigned)((size_t)R * nchunk);
    if (nwg >= 2u * (unsigned)cus)
      hipLaunchKernelGGL(select_chunk_kernel<512>, dim3(nwg), dim3(512), 0, s, beam_scores, logp, in, n, n_prev, n_cand,
                         nchunk, K, buf[which]);
    else
      hipLaunchKernelGGL(select_chunk_kernel<1024>, dim3(nwg), dim3(1024), 0, s, beam_scores, logp, in, n, n_prev,
                         n_cand, nchunk, K, buf[which]);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    in = buf[which];
    n = (long)nchunk * K;
    which ^= 1;
  }
  hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)R), dim3(kThreads), 0, s, beam_scores, logp, in, n, n_prev,
                     n_cand, K, parent, token, score);
  return hipGetLastError();
}

}  // namespace onela
