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
// Selection without sorting everything: an MSB-first radix select finds, among the keys held in LDS, the
// smallest key T such that exactly K keys are >= T (8-bit digits from the highest bit where the keys
// differ; it stops as soon as a whole digit bucket is taken).  The keys >= T are then compacted.
//   Reduce  workgroups of 8192 keys each keep their K best (unordered) in the caller's scratch buffer;
//           repeated until a request has at most 8192 keys left.  The first pass builds the keys from the
//           scores on the fly.
//   Final   one workgroup per request selects its K keys from the survivors (or straight from the scores
//           when there are few enough), orders them by counting ranks and writes parent, token, score.
// Key 0 pads short chunks and ranks below every real key.
#include "device_common.h"
#include "launchers.h"

namespace onela {

namespace {
constexpr int kRedChunk = 8192;   // keys per reduce workgroup
constexpr int kRedThreads = 1024;
constexpr int kFinalMax = 8192;   // keys one final workgroup holds in LDS
constexpr int kFinalThreads = 1024;
constexpr int kMaxBeams = 2048;

__device__ __forceinline__ uint32_t score_order(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t f) {
  return ((uint64_t)score_order(s) << 32) | (uint64_t)(~f);
}

// LDS scratch of the radix select: 256-bin histograms (one per wave, at most 8, shared round robin), the
// chosen digit, rank and bucket size, and the smallest and largest real key (key 0 is padding).
template <int NT>
struct SelShared {
  static constexpr int kCopies = NT / 64 < 8 ? NT / 64 : 8;
  int hist[kCopies][256];
  int digit, rank, count, n_out;
  unsigned long long kmin, kmax;
};

// Smallest key T such that exactly K of the n unique keys in `keys` are >= T (requires 1 <= K <= the number
// of nonzero keys).  Every thread of the workgroup must call it; NT is the workgroup size.  Digits start at
// the highest bit where the smallest and the largest real key differ: the bits above are common to all of
// them and would only cost passes that split nothing.
template <int NT>
__device__ uint64_t radix_threshold(const uint64_t* keys, int n, int K, SelShared<NT>& sh) {
  constexpr int kCopies = SelShared<NT>::kCopies;
  const int tid = threadIdx.x, lane = tid & 63, wv = (tid >> 6) % kCopies;
  unsigned long long lo = ~0ull, hi = 0ull;
  for (int i = tid; i < n; i += NT) {
    const unsigned long long k = keys[i];
    if (k != 0ull) {
      lo = k < lo ? k : lo;
      hi = k > hi ? k : hi;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long l2 = __shfl_xor(lo, off, 64), h2 = __shfl_xor(hi, off, 64);
    lo = l2 < lo ? l2 : lo;
    hi = h2 > hi ? h2 : hi;
  }
  if (tid == 0) {
    sh.kmin = ~0ull;
    sh.kmax = 0ull;
  }
  __syncthreads();
  if (lane == 0) {
    atomicMin(&sh.kmin, lo);
    atomicMax(&sh.kmax, hi);
  }
  __syncthreads();
  const uint64_t kmax = sh.kmax, diff = kmax ^ sh.kmin;
  if (diff == 0) return kmax;  // a single real key
  int top = 63 - __clzll((long long)diff);
  uint64_t mask = top == 63 ? 0ull : ~((2ull << top) - 1), prefix = kmax & mask;
  int rank = K;
  while (top >= 0) {
    const int w = top >= 7 ? 8 : top + 1, shift = top - w + 1;
    for (int i = tid; i < kCopies * 256; i += NT) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint64_t k = keys[i];
      if ((k & mask) == prefix) atomicAdd(&sh.hist[wv][(int)((k >> shift) & 0xFFu)], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255 - 4l .. 252 - 4l: lane order is descending digit order
      int c[4], local = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int v = 0;
        for (int x = 0; x < kCopies; ++x) v += sh.hist[x][255 - 4 * tid - e];
        c[e] = v;
        local += v;
      }
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
    const int d = sh.digit, cnt = sh.count;
    rank = sh.rank;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)((1u << w) - 1u) << shift;
    if (cnt == rank) break;  // the whole bucket is taken: exactly K keys are >= prefix
    top = shift - 1;
    __syncthreads();         // everyone has read the choice before the next pass rewrites it
  }
  return prefix;
}

// Write the keys >= thr (K of them) to out[0 .. K) in arbitrary order.
template <int NT>
__device__ void compact(const uint64_t* keys, int n, uint64_t thr, uint64_t* out, SelShared<NT>& sh) {
  if (threadIdx.x == 0) sh.n_out = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint64_t k = keys[i];
    const uint64_t take = __ballot(k >= thr);
    if (take) {  // one atomic per wave; lanes take consecutive places in lane order
      const int first = __ffsll((long long)take) - 1;
      int base = 0;
      if (lane == first) base = atomicAdd(&sh.n_out, __popcll(take));
      base = __shfl(base, first, 64);
      if (k >= thr) out[base + __popcll(take & ((1ull << lane) - 1))] = k;
    }
  }
  __syncthreads();
}

// Keys of chunk `c` of request r, padded with 0: built from the scores (in == nullptr) or copied from in.
template <int NT>
__device__ int load_keys(uint64_t* keys, int cap, const float* beam_scores, const float* logp,
                         const uint64_t* in, long n_in, int n_prev, int n_cand, int r, long base) {
  const int valid = (int)min((long)cap, n_in - base);
  if (in == nullptr) {
    const float* bs = beam_scores + (size_t)r * n_prev;
    const float* lp = logp + (size_t)r * n_in;
    for (int i = threadIdx.x; i < cap; i += NT) {
      uint64_t key = 0;
      if (i < valid) {
        const uint32_t f = (uint32_t)(base + i);
        key = make_key(bs[f / (uint32_t)n_cand] + lp[f], f);
      }
      keys[i] = key;
    }
  } else {
    const uint64_t* src = in + (size_t)r * n_in + base;
    for (int i = threadIdx.x; i < cap; i += NT) keys[i] = i < valid ? src[i] : 0ull;
  }
  __syncthreads();
  return valid;
}

__global__ __launch_bounds__(kRedThreads) void select_reduce_kernel(const float* __restrict__ beam_scores,
                                                                    const float* __restrict__ logp,
                                                                    const uint64_t* __restrict__ in, long n_in,
                                                                    int n_prev, int n_cand, int nchunk, int K,
                                                                    uint64_t* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);
  SelShared<kRedThreads>& sh = *reinterpret_cast<SelShared<kRedThreads>*>(keys + kRedChunk);
  const int r = blockIdx.x / nchunk, c = blockIdx.x - r * nchunk;
  const int valid = load_keys<kRedThreads>(keys, kRedChunk, beam_scores, logp, in, n_in, n_prev, n_cand, r,
                                           (long)c * kRedChunk);
  uint64_t* dst = out + ((size_t)r * nchunk + c) * K;
  if (valid <= K) {  // keep everything (the padding keys are 0)
    for (int i = threadIdx.x; i < K; i += kRedThreads) dst[i] = i < kRedChunk ? keys[i] : 0ull;
    return;
  }
  const uint64_t thr = radix_threshold<kRedThreads>(keys, kRedChunk, K, sh);
  compact<kRedThreads>(keys, kRedChunk, thr, dst, sh);
}

__global__ __launch_bounds__(kFinalThreads) void select_final_kernel(const float* __restrict__ beam_scores,
                                                                     const float* __restrict__ logp,
                                                                     const uint64_t* __restrict__ in, long n_in,
                                                                     int n_prev, int n_cand, int K,
                                                                     int32_t* parent, int32_t* token,
                                                                     float* score) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds);                 // n_in <= kFinalMax keys
  uint64_t* best = keys + kFinalMax;                                  // the K survivors, unordered
  SelShared<kFinalThreads>& sh = *reinterpret_cast<SelShared<kFinalThreads>*>(best + kMaxBeams);
  const int r = blockIdx.x;
  const int cap = (int)n_in;
  load_keys<kFinalThreads>(keys, cap, beam_scores, logp, in, n_in, n_prev, n_cand, r, 0);
  const uint64_t thr = radix_threshold<kFinalThreads>(keys, cap, K, sh);
  compact<kFinalThreads>(keys, cap, thr, best, sh);
  // order: the rank of a survivor is the number of survivors with a larger key (keys are unique, so the ranks
  // are a permutation of 0 .. K-1); every lane of a wave reads the same survivor at once (an LDS broadcast)
  uint64_t* sorted = keys;  // the candidate keys are no longer needed
  int* part = reinterpret_cast<int*>(keys + kMaxBeams);  // partial ranks: two threads per survivor
  constexpr int kPer = kFinalThreads / 2;
  for (int i0 = 0; i0 < K; i0 += kPer) {
    const int i = i0 + (threadIdx.x % kPer), half = threadIdx.x / kPer;
    const uint64_t mine = i < K ? best[i] : 0ull;
    const int j0 = half * (K / 2), j1 = half ? K : K / 2;
    int rank = 0, j = j0;
    for (; j + 16 <= j1; j += 16) {  // 16 survivors per iteration, 8 loads in flight
      u32x4_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = reinterpret_cast<const u32x4_t*>(best + j)[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint64_t a = ((uint64_t)w[u].y << 32) | w[u].x, b = ((uint64_t)w[u].w << 32) | w[u].z;
        rank += (a > mine ? 1 : 0) + (b > mine ? 1 : 0);
      }
    }
    for (; j < j1; ++j) rank += best[j] > mine ? 1 : 0;
    if (half == 1 && i < K) part[threadIdx.x % kPer] = rank;
    __syncthreads();
    if (half == 0 && i < K) sorted[rank + part[threadIdx.x]] = mine;
    __syncthreads();
  }
  // the score is recomputed from its inputs (the same float32 addition), so its sign survives
  const float* bs = beam_scores + (size_t)r * n_prev;
  const float* lp = logp + (size_t)r * n_prev * n_cand;
  for (int i = threadIdx.x; i < K; i += kFinalThreads) {
    const uint32_t f = ~(uint32_t)sorted[i];
    const uint32_t p = f / (uint32_t)n_cand;
    const size_t o = (size_t)r * K + i;
    parent[o] = (int32_t)p;
    token[o] = (int32_t)(f - p * (uint32_t)n_cand);
    score[o] = bs[p] + lp[f];
  }
}

size_t reduce_lds_bytes() { return (size_t)kRedChunk * sizeof(uint64_t) + sizeof(SelShared<kRedThreads>); }
size_t final_lds_bytes() {
  return (size_t)(kFinalMax + kMaxBeams) * sizeof(uint64_t) + sizeof(SelShared<kFinalThreads>);
}
}  // namespace

int beam_select_max_beams() { return kMaxBeams; }

size_t beam_select_scratch_bytes(int R, long n, int n_beams) {
  // keys surviving the first reduce pass, twice (later passes alternate between the two halves)
  if (n <= kFinalMax) return 0;
  const long nchunk = (n + kRedChunk - 1) / kRedChunk;
  return (size_t)2 * R * nchunk * n_beams * sizeof(uint64_t);
}

hipError_t launch_beam_select(const float* beam_scores, const float* logp, int R, int n_prev, int n_cand,
                              int n_beams, int32_t* parent, int32_t* token, float* score, void* scratch,
                              hipStream_t s) {
  long n = (long)n_prev * n_cand;
  const int K = n_beams;  // K <= kRedChunk / 4: every reduce pass at least quarters the keys
  uint64_t* buf[2] = {static_cast<uint64_t*>(scratch), nullptr};
  if (scratch) buf[1] = buf[0] + (size_t)R * ((n + kRedChunk - 1) / kRedChunk) * K;
  const uint64_t* in = nullptr;
  int which = 0;
  while (n > kFinalMax) {
    const int nchunk = (int)((n + kRedChunk - 1) / kRedChunk);
    const size_t rlds = reduce_lds_bytes();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_reduce_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)rlds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_reduce_kernel, dim3((unsigned)((size_t)R * nchunk)), dim3(kRedThreads), rlds, s,
                       beam_scores, logp, in, n, n_prev, n_cand, nchunk, K, buf[which]);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    in = buf[which];
    n = (long)nchunk * K;
    which ^= 1;
  }
  const size_t lds = final_lds_bytes();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_final_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_final_kernel, dim3((unsigned)R), dim3(kFinalThreads), lds, s, beam_scores, logp, in, n,
                     n_prev, n_cand, K, parent, token, score);
  return hipGetLastError();
}

}  // namespace onela
