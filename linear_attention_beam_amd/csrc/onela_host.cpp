// Host runtime of libonela: argument and state checks, workspace layout, kernel dispatch.
// The public contract (layouts, ownership, errors) is documented in include/onela.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "onela.h"
#include "launchers.h"

using namespace onela;

struct onela_ctx {
  onela_config cfg;
  unsigned char* ws;
  size_t ws_bytes;
  int device;
  bool fused;
  bool materialize;
  int* flag;
  float* sctx_t;
  uint16_t* sctx_frag;
  int32_t* chains;
  unsigned char* plan;  // fused path: per (request, beam tile) ancestry plans of the current step
  int tile;      // fused path: beams per tile
  int grid;      // fused path: persistent workgroups (compute units x workgroups per unit)
  void* rec_k;
  float* rec_u;
  float* rec_alpha;
  float* fullstate;
  unsigned char* scratch;  // the decode state (chains onwards): scratch of onela_prefill, which resets it
  size_t scratch_bytes;
  bool has_context;
  int t;
  int n_beams;
  int epoch;  // the device flag holds the epoch in which a bad parent was seen
  int max_lds;  // dynamic LDS bytes a workgroup may use on this device
};

namespace {

thread_local std::string g_last_error;

onela_status fail(onela_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

onela_status ok() {
  g_last_error.clear();
  return ONELA_OK;
}

struct Layout {
  size_t flag, sctx_t, sctx_frag, chains, plan, rec_k, rec_u, rec_alpha, fullstate, total;
  bool fused;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

onela_status check_config(const onela_config* c) {
  if (!c) return fail(ONELA_ERR_INVALID_ARG, "config is NULL");
  if (c->num_requests < 1 || c->num_heads < 1)
    return fail(ONELA_ERR_INVALID_ARG, "num_requests (%d) and num_heads (%d) must be >= 1", c->num_requests,
                c->num_heads);
  if (c->d_k < 1 || c->d_k > 256 || c->d_v < 1 || c->d_v > 256)
    return fail(ONELA_ERR_INVALID_ARG, "d_k (%d) and d_v (%d) must be in 1..256", c->d_k, c->d_v);
  if (c->max_beams < 1 || c->max_beams > (1 << 20))
    return fail(ONELA_ERR_INVALID_ARG, "max_beams (%d) must be in 1..2^20", c->max_beams);
  if (c->max_steps < 1 || c->max_steps > 64)
    return fail(ONELA_ERR_INVALID_ARG, "max_steps (%d) must be in 1..64", c->max_steps);
  if (c->qkv_dtype != ONELA_F32 && c->qkv_dtype != ONELA_BF16)
    return fail(ONELA_ERR_INVALID_ARG, "qkv_dtype %d is not ONELA_F32 or ONELA_BF16", c->qkv_dtype);
  if (c->mode != ONELA_MODE_REPLAY && c->mode != ONELA_MODE_FULLSTATE)
    return fail(ONELA_ERR_INVALID_ARG, "mode %d is not REPLAY or FULLSTATE", c->mode);
  if (c->flags & ~(ONELA_FLAG_FORCE_GENERIC | ONELA_FLAG_MATERIALIZE))
    return fail(ONELA_ERR_INVALID_ARG, "unknown flags 0x%x", c->flags);
  if (c->tile_beams != 0 && c->tile_beams != 16 && c->tile_beams != 32)
    return fail(ONELA_ERR_INVALID_ARG, "tile_beams %d is not 0, 16 or 32", c->tile_beams);
  const double slots_total =
      (double)c->num_requests * c->num_heads * (double)c->max_beams * c->max_steps * (c->d_k + c->d_v);
  if (slots_total > 9.0e15) return fail(ONELA_ERR_INVALID_ARG, "configuration too large");
  if ((double)c->num_requests * c->max_beams * c->num_heads > 2.0e9)
    return fail(ONELA_ERR_INVALID_ARG, "num_requests * max_beams * num_heads exceeds the launch grid");
  // per-(request, head) record arenas and per-request step inputs are addressed with 32-bit offsets
  if ((double)c->max_beams * c->max_steps * (c->d_k > c->d_v ? c->d_k : c->d_v) * 4.0 >= 2147483648.0 ||
      (double)c->max_beams * c->num_heads * (c->d_k > c->d_v ? c->d_k : c->d_v) * 4.0 >= 2147483648.0)
    return fail(ONELA_ERR_INVALID_ARG, "max_beams * max_steps * d or max_beams * num_heads * d exceeds 2^31 bytes");
  return ONELA_OK;
}

Layout make_layout(const onela_config* c) {
  Layout l{};
  const size_t R = c->num_requests, H = c->num_heads, dk = c->d_k, dv = c->d_v;
  const size_t B = c->max_beams, L = c->max_steps, slots = B * L;
  const size_t in_bytes = c->qkv_dtype == ONELA_BF16 ? 2 : 4;
  l.fused = c->mode == ONELA_MODE_REPLAY && c->qkv_dtype == ONELA_BF16 && !(c->flags & (ONELA_FLAG_FORCE_GENERIC | ONELA_FLAG_MATERIALIZE)) &&
            fused_supported(c->d_k, c->d_v, c->max_steps);
  size_t off = 0;
  l.flag = off;       off += 256;
  l.sctx_t = off;     off = align256(off + R * H * dk * dv * 4);
  l.sctx_frag = off;  off = align256(off + (l.fused ? R * H * dk * dv * 2 * 2 : 0));
  l.chains = off;     off = align256(off + L * R * B * L * 4);
  l.plan = off;       off = align256(off + (l.fused ? fused_plan_bytes((int)R, (int)B, (int)L) : 0));
  if (c->mode == ONELA_MODE_REPLAY) {
    l.rec_k = off;     off = align256(off + R * H * slots * dk * in_bytes);
    l.rec_u = off;     off = align256(off + R * H * slots * dv * 4);
    l.rec_alpha = off; off = align256(off + R * H * slots * 4);
    l.fullstate = 0;
  } else {
    l.rec_k = l.rec_u = l.rec_alpha = 0;
    l.fullstate = off; off = align256(off + 2 * R * H * B * dk * dv * 4);
  }
  l.total = off;
  return l;
}

onela_status check_handle(onela_handle h) {
  if (!h) return fail(ONELA_ERR_INVALID_ARG, "handle is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ONELA_ERR_DEVICE, "hipGetDevice failed");
  if (dev != h->device)
    return fail(ONELA_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev, h->device);
  return ONELA_OK;
}

onela_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ONELA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ONELA_OK;
}

// Split the transposed state already in the workspace into the fused kernel's bf16 fragments.
onela_status finish_context(onela_handle h, hipStream_t s) {
  const onela_config& c = h->cfg;
  if (h->fused) {
    onela_status st =
        launched(launch_split_frag(h->sctx_t, h->sctx_frag, c.num_requests * c.num_heads, c.d_v, c.d_k, s),
                 "split of S_ctx");
    if (st != ONELA_OK) return st;
  }
  onela_status st = launched(launch_clear_flag(h->flag, s), "flag reset");
  if (st != ONELA_OK) return st;
  h->has_context = true;
  h->t = 0;
  h->n_beams = 1;
  h->epoch += 1;
  return ok();
}

}  // namespace

extern "C" {

onela_status onela_workspace_size(const onela_config* cfg, size_t* bytes) {
  onela_status st = check_config(cfg);
  if (st != ONELA_OK) return st;
  if (!bytes) return fail(ONELA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_layout(cfg).total;
  return ok();
}

onela_status onela_create(const onela_config* cfg, void* d_workspace, size_t workspace_bytes, onela_handle* out) {
  onela_status st = check_config(cfg);
  if (st != ONELA_OK) return st;
  if (!out) return fail(ONELA_ERR_INVALID_ARG, "out is NULL");
  if (!d_workspace) return fail(ONELA_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_workspace) & 255)
    return fail(ONELA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const Layout l = make_layout(cfg);
  if (workspace_bytes < l.total)
    return fail(ONELA_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", workspace_bytes, l.total);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(ONELA_ERR_DEVICE, "hipGetDevice failed");
  int max_lds = 0;
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return fail(ONELA_ERR_DEVICE, "hipDeviceGetAttribute failed");
  onela_ctx* h = new (std::nothrow) onela_ctx{};
  if (!h) return fail(ONELA_ERR_CAPACITY, "out of host memory");
  unsigned char* ws = static_cast<unsigned char*>(d_workspace);
  h->cfg = *cfg;
  h->ws = ws;
  h->ws_bytes = workspace_bytes;
  h->device = dev;
  h->fused = l.fused;
  h->materialize = cfg->mode == ONELA_MODE_REPLAY && (cfg->flags & ONELA_FLAG_MATERIALIZE);
  h->flag = reinterpret_cast<int*>(ws + l.flag);
  h->sctx_t = reinterpret_cast<float*>(ws + l.sctx_t);
  h->sctx_frag = l.fused ? reinterpret_cast<uint16_t*>(ws + l.sctx_frag) : nullptr;
  h->chains = reinterpret_cast<int32_t*>(ws + l.chains);
  h->plan = l.fused ? ws + l.plan : nullptr;
  h->tile = 0;
  h->grid = 0;
  if (l.fused) {
    h->tile = fused_pick_tile(cfg->d_k, cfg->d_v, cfg->max_steps, cfg->tile_beams);
    const size_t lds = fused_lds_bytes(h->tile, cfg->max_steps, cfg->d_k, cfg->d_v);
    if (lds > (size_t)max_lds) {
      delete h;
      return fail(ONELA_ERR_UNSUPPORTED, "tile_beams %d with max_steps %d needs %zu bytes of LDS, the device allows %d",
                  h->tile, cfg->max_steps, lds, max_lds);
    }
    const hipError_t e = fused_prepare(h->tile, cfg->d_k, cfg->d_v, cfg->max_steps, &h->grid);
    if (e != hipSuccess) {
      delete h;
      return fail(ONELA_ERR_DEVICE, "fused kernel set-up: %s", hipGetErrorString(e));
    }
  }
  if (cfg->mode == ONELA_MODE_REPLAY) {
    h->rec_k = ws + l.rec_k;
    h->rec_u = reinterpret_cast<float*>(ws + l.rec_u);
    h->rec_alpha = reinterpret_cast<float*>(ws + l.rec_alpha);
    h->fullstate = nullptr;
  } else {
    h->rec_k = nullptr;
    h->rec_u = h->rec_alpha = nullptr;
    h->fullstate = reinterpret_cast<float*>(ws + l.fullstate);
  }
  h->scratch = ws + l.chains;
  h->scratch_bytes = l.total - l.chains;
  h->has_context = false;
  h->t = 0;
  h->n_beams = 1;
  h->epoch = 0;
  h->max_lds = max_lds;
  *out = h;
  return ok();
}

onela_status onela_destroy(onela_handle h) {
  if (!h) return fail(ONELA_ERR_INVALID_ARG, "handle is NULL");
  delete h;
  return ok();
}

onela_status onela_set_context(onela_handle h, const float* d_sctx, void* stream) {
  onela_status st = check_handle(h);
  if (st != ONELA_OK) return st;
  if (!d_sctx) return fail(ONELA_ERR_INVALID_ARG, "S_ctx is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const onela_config& c = h->cfg;
  st = launched(launch_transpose_sctx(d_sctx, h->sctx_t, c.num_requests * c.num_heads, c.d_v, c.d_k, s),
                "transpose of S_ctx");
  if (st != ONELA_OK) return st;
  return finish_context(h, s);
}

onela_status onela_prefill(onela_handle h, int32_t n_tokens, const float* d_k, const float* d_v,
                           const float* d_alpha, const float* d_beta, float* d_sctx_out, void* stream) {
  onela_status st = check_handle(h);
  if (st != ONELA_OK) return st;
  const onela_config& c = h->cfg;
  if (n_tokens < 0) return fail(ONELA_ERR_INVALID_ARG, "n_tokens (%d) must be >= 0", n_tokens);
  if (n_tokens > 0 && (!d_k || !d_v || !d_alpha || !d_beta))
    return fail(ONELA_ERR_INVALID_ARG, "prefill inputs must not be NULL");
  if (!prefill_supported(c.d_k, c.d_v))
    return fail(ONELA_ERR_UNSUPPORTED, "prefill supports d_k, d_v <= 256 (d_k=%d, d_v=%d)", c.d_k, c.d_v);
  if ((double)c.num_requests * n_tokens * c.num_heads * (c.d_k > c.d_v ? c.d_k : c.d_v) > 9.0e15)
    return fail(ONELA_ERR_INVALID_ARG, "prompt too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launched(launch_prefill(d_k, d_v, d_alpha, d_beta, c.num_requests, c.num_heads, n_tokens, c.d_k, c.d_v,
                               h->sctx_t, d_sctx_out, h->scratch, h->scratch_bytes, s),
                "prefill");
  if (st != ONELA_OK) return st;
  return finish_context(h, s);
}

onela_status onela_step(onela_handle h, int32_t n_beams, const void* d_q, const void* d_k, const void* d_v,
                        const float* d_alpha, const float* d_beta, const int32_t* d_parent_idx, float* d_o,
                        void* stream) {
  onela_status st = check_handle(h);
  if (st != ONELA_OK) return st;
  const onela_config& c = h->cfg;
  if (!h->has_context) return fail(ONELA_ERR_STATE, "no context: call onela_set_context or onela_prefill first");
  if (h->t >= c.max_steps) return fail(ONELA_ERR_CAPACITY, "all %d steps of this context are used", c.max_steps);
  if (n_beams < 1 || n_beams > c.max_beams)
    return fail(ONELA_ERR_INVALID_ARG, "n_beams (%d) must be in 1..max_beams (%d)", n_beams, c.max_beams);
  if (!d_q || !d_k || !d_v || !d_alpha || !d_beta || !d_parent_idx || !d_o)
    return fail(ONELA_ERR_INVALID_ARG, "a step buffer is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int t = h->t + 1;
  const size_t table = (size_t)c.num_requests * c.max_beams * c.max_steps;
  const int32_t* chain_prev = t == 1 ? nullptr : h->chains + (size_t)(t - 2) * table;
  int32_t* chain_out = h->chains + (size_t)(t - 1) * table;
  if (c.mode == ONELA_MODE_FULLSTATE || !h->fused) {  // the fused kernel updates the index itself
    st = launched(launch_ancestry(d_parent_idx, chain_prev, chain_out, c.num_requests, n_beams, h->n_beams,
                                  c.max_beams, c.max_steps, t, h->flag, h->epoch, s),
                  "ancestry update");
    if (st != ONELA_OK) return st;
  }

  StepArgs a{};
  a.q = d_q; a.k = d_k; a.v = d_v; a.alpha = d_alpha; a.beta = d_beta; a.o = d_o;
  a.sctx_t = h->sctx_t;
  a.sctx_frag = h->sctx_frag;
  a.rec_k = h->rec_k; a.rec_u = h->rec_u; a.rec_alpha = h->rec_alpha;
  a.chain = chain_out;
  a.parent = d_parent_idx; a.chain_prev = chain_prev; a.chain_out = chain_out;
  a.flag = h->flag; a.epoch = h->epoch; a.b_prev = h->n_beams;
  a.R = c.num_requests; a.H = c.num_heads; a.d_k = c.d_k; a.d_v = c.d_v; a.n = n_beams;
  a.B_max = c.max_beams; a.L_max = c.max_steps; a.slots = c.max_beams * c.max_steps; a.t = t;
  const bool bf16 = c.qkv_dtype == ONELA_BF16;
  if (c.mode == ONELA_MODE_FULLSTATE) {
    const size_t buf = (size_t)c.num_requests * c.num_heads * c.max_beams * c.d_k * c.d_v;
    const float* prev = h->fullstate + (size_t)((t - 1) & 1) * buf;
    float* next = h->fullstate + (size_t)(t & 1) * buf;
    st = launched(launch_fullstate(a, bf16, d_parent_idx, h->n_beams, prev, next, s), "FullState step");
  } else if (h->fused) {
    st = launched(launch_step_fused(a, h->tile, h->plan, h->grid, s), "fused step");
  } else {
    st = h->materialize ? launched(launch_step_materialize(a, bf16, s), "materializing step")
                        : launched(launch_step_generic(a, bf16, s), "step");
  }
  if (st != ONELA_OK) return st;
  h->t = t;
  h->n_beams = n_beams;
  return ok();
}

onela_status onela_reset(onela_handle h, void* stream) {
  (void)stream;  // nothing to enqueue: records and chains are overwritten by the next steps, and a new
                 // epoch retires any bad-parent flag of the previous decode
  onela_status st = check_handle(h);
  if (st != ONELA_OK) return st;
  h->t = 0;
  h->n_beams = 1;
  h->epoch += 1;
  return ok();
}

onela_status onela_get_status(onela_handle h, void* stream) {
  onela_status st = check_handle(h);
  if (st != ONELA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int flag = 0;
  if (hipMemcpyAsync(&flag, h->flag, sizeof flag, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(ONELA_ERR_DEVICE, "reading the device flag failed: %s", hipGetErrorString(hipGetLastError()));
  if (h->has_context && flag == h->epoch) return fail(ONELA_ERR_BAD_PARENT, "a parent index was out of range");
  return ok();
}

onela_status onela_get_view(onela_handle h, onela_view* view) {
  if (!h || !view) return fail(ONELA_ERR_INVALID_ARG, "handle or view is NULL");
  view->t = h->t;
  view->n_beams = h->n_beams;
  view->slots = h->cfg.max_beams * h->cfg.max_steps;
  view->fused = h->fused ? 1 : 0;
  view->rec_k = h->rec_k;
  view->rec_u = h->rec_u;
  view->rec_alpha = h->rec_alpha;
  view->chains = h->chains;
  view->sctx_t = h->sctx_t;
  view->fullstate = h->fullstate;
  return ok();
}

static onela_status select_args(int32_t R, int32_t n_prev, int32_t n_cand, int32_t n_beams) {
  if (R < 1 || n_prev < 1 || n_cand < 1 || n_beams < 1)
    return fail(ONELA_ERR_INVALID_ARG, "num_requests (%d), n_prev (%d), n_cand (%d) and n_beams (%d) must be >= 1",
                R, n_prev, n_cand, n_beams);
  const long n = (long)n_prev * n_cand;
  if (n >= 2147483648L) return fail(ONELA_ERR_INVALID_ARG, "n_prev * n_cand (%ld) must be below 2^31", n);
  if (n_beams > n) return fail(ONELA_ERR_INVALID_ARG, "n_beams (%d) exceeds the %ld candidates", n_beams, n);
  if (n_beams > beam_select_max_beams())
    return fail(ONELA_ERR_UNSUPPORTED, "n_beams (%d) above %d", n_beams, beam_select_max_beams());
  if ((double)R * n >= 9.0e15) return fail(ONELA_ERR_INVALID_ARG, "selection too large");
  return ONELA_OK;
}

onela_status onela_beam_select_scratch(int32_t num_requests, int32_t n_prev, int32_t n_cand, int32_t n_beams,
                                       size_t* bytes) {
  if (!bytes) return fail(ONELA_ERR_INVALID_ARG, "bytes is NULL");
  const onela_status st = select_args(num_requests, n_prev, n_cand, n_beams);
  if (st != ONELA_OK) return st;
  *bytes = beam_select_scratch_bytes(num_requests, (long)n_prev * n_cand, n_beams);
  return ok();
}

onela_status onela_beam_select(int32_t num_requests, int32_t n_prev, int32_t n_cand, int32_t n_beams,
                               const float* d_beam_scores, const float* d_logp, int32_t* d_parent_idx,
                               int32_t* d_token, float* d_scores, void* d_scratch, size_t scratch_bytes,
                               void* stream) {
  onela_status st = select_args(num_requests, n_prev, n_cand, n_beams);
  if (st != ONELA_OK) return st;
  if (!d_beam_scores || !d_logp || !d_parent_idx || !d_token || !d_scores)
    return fail(ONELA_ERR_INVALID_ARG, "a beam-selection buffer is NULL");
  const size_t need = beam_select_scratch_bytes(num_requests, (long)n_prev * n_cand, n_beams);
  if (need > 0 && (!d_scratch || scratch_bytes < need))
    return fail(ONELA_ERR_INVALID_ARG, "scratch of %zu bytes is smaller than the %zu required", scratch_bytes, need);
  st = launched(launch_beam_select(d_beam_scores, d_logp, num_requests, n_prev, n_cand, n_beams, d_parent_idx,
                                   d_token, d_scores, need > 0 ? d_scratch : nullptr,
                                   static_cast<hipStream_t>(stream)),
                "beam selection");
  return st != ONELA_OK ? st : ok();
}

onela_status onela_beam_select_noalloc(int32_t num_requests, int32_t n_prev, int32_t n_cand, int32_t n_beams,
                                       const float* d_beam_scores, const float* d_logp, int32_t* d_parent_idx,
                                       int32_t* d_token, float* d_scores, void* stream) {
  onela_status st = select_args(num_requests, n_prev, n_cand, n_beams);
  if (st != ONELA_OK) return st;
  if (!d_beam_scores || !d_logp || !d_parent_idx || !d_token || !d_scores)
    return fail(ONELA_ERR_INVALID_ARG, "a beam-selection buffer is NULL");
  const size_t need = beam_select_scratch_bytes(num_requests, (long)n_prev * n_cand, n_beams);
  if (need > beam_select_static_max())
    return fail(ONELA_ERR_CAPACITY, "selection needs %zu bytes of scratch, above the %zu the library holds", need,
                beam_select_static_max());
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = beam_select_static_scratch(&scratch);
    if (e != hipSuccess) return fail(ONELA_ERR_DEVICE, "static scratch lookup: %s", hipGetErrorString(e));
  }
  st = launched(launch_beam_select(d_beam_scores, d_logp, num_requests, n_prev, n_cand, n_beams, d_parent_idx,
                                   d_token, d_scores, scratch, static_cast<hipStream_t>(stream)),
                "beam selection");
  return st != ONELA_OK ? st : ok();
}

const char* onela_status_string(onela_status s) {
  switch (s) {
    case ONELA_OK: return "ONELA_OK";
    case ONELA_ERR_INVALID_ARG: return "ONELA_ERR_INVALID_ARG";
    case ONELA_ERR_STATE: return "ONELA_ERR_STATE";
    case ONELA_ERR_CAPACITY: return "ONELA_ERR_CAPACITY";
    case ONELA_ERR_DEVICE: return "ONELA_ERR_DEVICE";
    case ONELA_ERR_BAD_PARENT: return "ONELA_ERR_BAD_PARENT";
    case ONELA_ERR_UNSUPPORTED: return "ONELA_ERR_UNSUPPORTED";
  }
  return "unknown onela_status";
}

const char* onela_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
