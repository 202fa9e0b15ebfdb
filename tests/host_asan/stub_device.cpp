// Host stand-ins for the HIP runtime calls and the kernel launchers of the library, for a sanitizer build of
// onela_host.cpp without a GPU.  Each launcher touches, in host memory, exactly the buffer extents the real
// kernel reads and writes (so that AddressSanitizer sees any region the host code sizes or places wrongly),
// and the parent checks raise the sticky flag the way the device code does.  Test infrastructure only.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <utility>
#include <vector>

#include "launchers.h"

int g_stub_device = 0;              // what hipGetDevice reports
int g_stub_fail_launch = 0;         // when nonzero, the next launcher fails once
long g_stub_launches = 0;           // launchers called
static hipError_t g_last = hipSuccess;

hipError_t hipGetDevice(int* device) {
  *device = g_stub_device;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  *value = attr == hipDeviceAttributeMaxSharedMemoryPerBlock ? 160 * 1024 : 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "stub launch failure"; }
hipError_t hipGetLastError() {
  const hipError_t e = g_last;
  g_last = hipSuccess;
  return e;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  std::memmove(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

namespace {
volatile unsigned char g_sink;
// read every byte of [p, p + bytes)
void touch_read(const void* p, size_t bytes) {
  const unsigned char* c = static_cast<const unsigned char*>(p);
  unsigned char x = 0;
  for (size_t i = 0; i < bytes; ++i) x ^= c[i];
  g_sink = x;
}
// Bounding range of everything written per kind of buffer since the last stub_extents_reset(): regions of one
// workspace that the host placed on top of each other show up as overlapping ranges.
enum Kind { kFlag, kSctx, kFrag, kChains, kPlan, kRecK, kRecU, kRecAlpha, kFullState, kScratch, kOut };
std::map<int, std::pair<uintptr_t, uintptr_t>> g_extent;
// overwrite [p, p + bytes) with a pattern
void touch_write(void* p, size_t bytes, Kind kind = kOut) {
  std::memset(p, 0x5A, bytes);
  if (!bytes) return;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p), hi = lo + bytes;
  auto it = g_extent.find(kind);
  if (it == g_extent.end()) {
    g_extent[kind] = {lo, hi};
  } else {
    it->second.first = std::min(it->second.first, lo);
    it->second.second = std::max(it->second.second, hi);
  }
}

hipError_t launched() {
  ++g_stub_launches;
  if (g_stub_fail_launch) {
    g_stub_fail_launch = 0;
    g_last = hipErrorLaunchFailure;
    return hipErrorLaunchFailure;
  }
  return hipSuccess;
}

// chain table after step t from the parents, with the device's range check
void ancestry(const int32_t* parent, const int32_t* chain_prev, int32_t* chain_out, int R, int n, int b_prev,
              int B_max, int L_max, int t, int* flag, int epoch) {
  for (int r = 0; r < R; ++r)
    for (int b = 0; b < B_max; ++b) {
      int32_t* out = chain_out + ((size_t)r * B_max + b) * L_max;
      if (b >= n) {
        for (int m = 0; m < L_max; ++m) out[m] = -1;
        continue;
      }
      int p = parent[(size_t)r * n + b];
      if (p < 0 || p >= b_prev) {
        *flag = epoch;
        p = 0;
      }
      for (int m = 0; m < L_max; ++m) {
        int32_t v = -1;
        if (m < t - 1) v = chain_prev[((size_t)r * B_max + p) * L_max + m];
        if (m == t - 1) v = (t - 1) * B_max + b;
        out[m] = v;
      }
    }
  touch_write(chain_out, 0, kChains);
  auto it = g_extent.find(kChains);
  const uintptr_t lo = reinterpret_cast<uintptr_t>(chain_out), hi = lo + (size_t)R * B_max * L_max * 4;
  if (it == g_extent.end()) g_extent[kChains] = {lo, hi};
  else {
    it->second.first = std::min(it->second.first, lo);
    it->second.second = std::max(it->second.second, hi);
  }
}

// what every replay step reads and writes besides the chain table
void step_io(const onela::StepArgs& a, bool bf16) {
  const size_t in = bf16 ? 2 : 4, rows = (size_t)a.R * a.n * a.H;
  touch_read(a.q, rows * a.d_k * in);
  touch_read(a.k, rows * a.d_k * in);
  touch_read(a.v, rows * a.d_v * in);
  touch_read(a.alpha, rows * 4);
  touch_read(a.beta, rows * 4);
  touch_read(a.parent, (size_t)a.R * a.n * 4);
  touch_write(a.o, rows * a.d_v * 4);
  touch_read(a.sctx_t, (size_t)a.R * a.H * a.d_k * a.d_v * 4);
  if (a.rec_k) {
    // the new records at slot (t - 1) * B_max + b, and every older record as the replay may read it
    for (size_t rh = 0; rh < (size_t)a.R * a.H; ++rh) {
      const size_t arena = rh * a.slots;
      touch_read(static_cast<const unsigned char*>(a.rec_k) + arena * a.d_k * in, (size_t)(a.t - 1) * a.B_max * a.d_k * in);
      touch_read(a.rec_u + arena * a.d_v, (size_t)(a.t - 1) * a.B_max * a.d_v * 4);
      touch_read(a.rec_alpha + arena, (size_t)(a.t - 1) * a.B_max * 4);
      const size_t own = arena + (size_t)(a.t - 1) * a.B_max;
      touch_write(static_cast<unsigned char*>(a.rec_k) + own * a.d_k * in, (size_t)a.n * a.d_k * in, kRecK);
      touch_write(a.rec_u + own * a.d_v, (size_t)a.n * a.d_v * 4, kRecU);
      touch_write(a.rec_alpha + own, (size_t)a.n * 4, kRecAlpha);
    }
  }
}
}  // namespace

void stub_extents_reset() { g_extent.clear(); }
// true when no two kinds of workspace buffer were written over the same bytes
bool stub_extents_disjoint() {
  bool ok = true;
  for (auto a = g_extent.begin(); a != g_extent.end(); ++a)
    for (auto b = std::next(a); b != g_extent.end(); ++b)
      if (a->first != kOut && b->first != kOut && a->second.first < b->second.second &&
          b->second.first < a->second.second) {
        std::fprintf(stderr, "buffer kinds %d and %d overlap\n", a->first, b->first);
        ok = false;
      }
  return ok;
}

namespace onela {

hipError_t launch_ancestry(const int32_t* parent, const int32_t* chain_prev, int32_t* chain_out, int R, int n,
                           int b_prev, int B_max, int L_max, int t, int* flag, int epoch, hipStream_t) {
  ancestry(parent, chain_prev, chain_out, R, n, b_prev, B_max, L_max, t, flag, epoch);
  return launched();
}
hipError_t launch_clear_flag(int* flag, hipStream_t) {
  flag[0] = 0;
  touch_write(flag, 4, kFlag);
  return launched();
}
hipError_t launch_transpose_sctx(const float* S, float* ST, int RH, int d_v, int d_k, hipStream_t) {
  touch_read(S, (size_t)RH * d_v * d_k * 4);
  touch_write(ST, (size_t)RH * d_v * d_k * 4, kSctx);
  return launched();
}
hipError_t launch_split_frag(const float* ST, uint16_t* frag, int RH, int d_v, int d_k, hipStream_t) {
  touch_read(ST, (size_t)RH * d_v * d_k * 4);
  touch_write(frag, (size_t)RH * d_v * d_k * 2 * 2, kFrag);
  return launched();
}
bool prefill_supported(int d_k, int d_v) { return d_k <= 256 && d_v <= 256; }
bool prefill_mfma_supported(int d_k, int d_v) { return d_k == 128 && (d_v == 16 || d_v == 32 || d_v == 64 || d_v == 128 || d_v == 256); }
size_t prefill_mfma_chunk_bytes(int R, int H) { return (size_t)R * H * 4480; }
hipError_t launch_prefill(const float* k, const float* v, const float* alpha, const float* beta, int R, int H, int N,
                          int d_k, int d_v, float* sctx_t, float* sctx_out, void* scratch, size_t scratch_bytes,
                          hipStream_t) {
  const size_t rows = (size_t)R * N * H;
  if (N > 0) {
    touch_read(k, rows * d_k * 4);
    touch_read(v, rows * d_v * 4);
    touch_read(alpha, rows * 4);
    touch_read(beta, rows * 4);
  }
  touch_write(sctx_t, (size_t)R * H * d_k * d_v * 4, kSctx);
  if (sctx_out) touch_write(sctx_out, (size_t)R * H * d_k * d_v * 4);
  touch_write(scratch, scratch_bytes, kScratch);
  return launched();
}
hipError_t launch_prefill_mfma(const float*, const float*, const float*, const float*, int, int, int, int, float*,
                               float*, void*, size_t, hipStream_t) {
  return launched();
}
hipError_t launch_step_generic(const StepArgs& a, bool bf16, hipStream_t) {
  step_io(a, bf16);
  touch_read(a.chain, (size_t)a.R * a.B_max * a.L_max * 4);
  return launched();
}
hipError_t launch_step_materialize(const StepArgs& a, bool bf16, hipStream_t) {
  step_io(a, bf16);
  touch_read(a.chain, (size_t)a.R * a.B_max * a.L_max * 4);
  return launched();
}

bool fused_supported(int d_k, int d_v, int L_max) {
  return (d_k == 128 || d_k == 64 || d_k == 256) && d_v % 32 == 0 && d_v >= 32 && L_max <= 64;
}
int fused_pick_tile(int, int, int, int requested) { return requested ? requested : 32; }
size_t fused_lds_bytes(int tile, int L_max, int d_k, int d_v) {
  return (size_t)tile * (6 * d_k + 9 * L_max) + 64 * 6 * d_k + d_v;
}
size_t fused_plan_bytes(int R, int B_max, int L_max) {
  return (size_t)R * ((B_max + 15) / 16) * (272 + 64 + 16 * L_max) + (size_t)R * B_max * 4;
}
hipError_t fused_prepare(int, int, int, int, int* grid) {
  *grid = 512;
  return hipSuccess;
}
hipError_t launch_step_fused(const StepArgs& a, int, void* plan, int, hipStream_t) {
  // the fused path derives the chain table itself (plan kernel, or the step-1 rows)
  if (a.t > 1) touch_write(plan, fused_plan_bytes(a.R, a.B_max, a.L_max), kPlan);
  ancestry(a.parent, a.chain_prev, a.chain_out, a.R, a.n, a.b_prev, a.B_max, a.L_max, a.t, a.flag, a.epoch);
  touch_read(a.sctx_frag, (size_t)a.R * a.H * a.d_k * a.d_v * 2 * 2);
  step_io(a, true);
  return launched();
}

int beam_select_max_beams() { return 2048; }
size_t beam_select_scratch_bytes(int R, long n, int n_beams) {
  if (n <= 8192) return 0;
  return (size_t)2 * R * ((n + 8191) / 8192) * n_beams * 8;
}
hipError_t launch_beam_select(const float* beam_scores, const float* logp, int R, int n_prev, int n_cand, int n_beams,
                              int32_t* parent, int32_t* token, float* score, void* scratch, hipStream_t) {
  touch_read(beam_scores, (size_t)R * n_prev * 4);
  touch_read(logp, (size_t)R * n_prev * n_cand * 4);
  const size_t need = beam_select_scratch_bytes(R, (long)n_prev * n_cand, n_beams);
  if (need) touch_write(scratch, need);
  for (size_t i = 0; i < (size_t)R * n_beams; ++i) {
    parent[i] = 0;
    token[i] = (int32_t)(i % n_cand);
    score[i] = 0.f;
  }
  return launched();
}
static std::vector<unsigned char> g_static_scratch(size_t(8) << 20);
size_t beam_select_static_max() { return g_static_scratch.size(); }
hipError_t beam_select_static_scratch(void** ptr) {
  *ptr = g_static_scratch.data();
  return hipSuccess;
}
hipError_t launch_fullstate(const StepArgs& a, bool bf16, const int32_t* parent, int b_prev, const float* fs_prev,
                            float* fs_next, hipStream_t) {
  const size_t buf = (size_t)a.R * a.H * a.B_max * a.d_k * a.d_v * 4;
  touch_read(parent, (size_t)a.R * a.n * 4);
  (void)b_prev;
  touch_read(fs_prev, buf);
  touch_write(fs_next, (size_t)a.R * a.H * a.n * a.d_k * a.d_v * 4, kFullState);
  const size_t in = bf16 ? 2 : 4, rows = (size_t)a.R * a.n * a.H;
  touch_read(a.q, rows * a.d_k * in);
  touch_write(a.o, rows * a.d_v * 4);
  return launched();
}

}  // namespace onela
