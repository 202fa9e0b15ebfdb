// State machine and argument checks of the C ABI (include/onela.h), run against host stand-ins of the device
// (stub_device.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.  Exit status 0 when every check
// holds.  Test infrastructure only.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "onela.h"

extern int g_stub_device;
extern int g_stub_fail_launch;
void stub_extents_reset();
bool stub_extents_disjoint();

static int g_failures = 0;
#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                             \
    }                                                                           \
  } while (0)
#define EXPECT_ST(call, want) EXPECT((call) == (want))

namespace {

onela_config make(int R, int H, int dk, int dv, int B, int L, int dtype, int mode, int flags, int tile) {
  onela_config c{};
  c.num_requests = R;
  c.num_heads = H;
  c.d_k = dk;
  c.d_v = dv;
  c.max_beams = B;
  c.max_steps = L;
  c.qkv_dtype = dtype;
  c.mode = mode;
  c.flags = flags;
  c.tile_beams = tile;
  return c;
}

// A buffer of exactly `bytes` (so the sanitizer sees its true end), 256-byte aligned.
struct Buf {
  void* p = nullptr;
  explicit Buf(size_t bytes) {
    const size_t n = bytes ? bytes : 1;
    if (posix_memalign(&p, 256, n) != 0) {
      std::fprintf(stderr, "out of host memory\n");
      std::exit(2);
    }
    std::memset(p, 0, n);
  }
  ~Buf() { std::free(p); }
  template <class T> T* as() { return static_cast<T*>(p); }
};

// One decode context driven through its whole life: errors before a context, steps to capacity, reset,
// bad parents, prefill, views.
void run_context(const onela_config& c) {
  size_t ws_bytes = 0;
  EXPECT_ST(onela_workspace_size(&c, &ws_bytes), ONELA_OK);
  size_t again = 0;
  EXPECT_ST(onela_workspace_size(&c, &again), ONELA_OK);
  EXPECT(again == ws_bytes && ws_bytes % 256 == 0);
  Buf ws(ws_bytes);
  onela_handle h = nullptr;
  EXPECT_ST(onela_create(&c, ws.p, ws_bytes - 256, &h), ONELA_ERR_CAPACITY);
  EXPECT_ST(onela_create(&c, static_cast<char*>(ws.p) + 16, ws_bytes, &h), ONELA_ERR_INVALID_ARG);
  EXPECT_ST(onela_create(&c, nullptr, ws_bytes, &h), ONELA_ERR_INVALID_ARG);
  EXPECT_ST(onela_create(&c, ws.p, ws_bytes, nullptr), ONELA_ERR_INVALID_ARG);
  EXPECT_ST(onela_create(&c, ws.p, ws_bytes, &h), ONELA_OK);
  if (!h) return;
  stub_extents_reset();

  const int R = c.num_requests, H = c.num_heads, dk = c.d_k, dv = c.d_v, B = c.max_beams, L = c.max_steps;
  const size_t in = c.qkv_dtype == ONELA_BF16 ? 2 : 4;
  Buf q((size_t)R * B * H * dk * in), k((size_t)R * B * H * dk * in), v((size_t)R * B * H * dv * in);
  Buf al((size_t)R * B * H * 4), be((size_t)R * B * H * 4), o((size_t)R * B * H * dv * 4);
  Buf par((size_t)R * B * 4), sctx((size_t)R * H * dv * dk * 4);
  int32_t* parent = par.as<int32_t>();

  // no context yet
  EXPECT_ST(onela_step(h, 1, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr),
            ONELA_ERR_STATE);
  EXPECT_ST(onela_get_status(h, nullptr), ONELA_OK);
  EXPECT(std::strlen(onela_last_error()) == 0);  // a successful call clears the message
  EXPECT_ST(onela_set_context(h, nullptr, nullptr), ONELA_ERR_INVALID_ARG);
  EXPECT(std::strlen(onela_last_error()) > 0);
  EXPECT_ST(onela_set_context(h, sctx.as<float>(), nullptr), ONELA_OK);

  // steps 1..L with a varying beam count, all parents valid
  for (int round = 0; round < 2; ++round) {
    int b_prev = 1;
    for (int t = 1; t <= L; ++t) {
      const int n = 1 + (t * 7 + round) % B;
      for (int r = 0; r < R; ++r)
        for (int b = 0; b < n; ++b) parent[(size_t)r * n + b] = (b * 5 + r) % b_prev;
      EXPECT_ST(onela_step(h, 0, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr),
                ONELA_ERR_INVALID_ARG);
      EXPECT_ST(onela_step(h, B + 1, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr),
                ONELA_ERR_INVALID_ARG);
      EXPECT_ST(onela_step(h, n, q.p, nullptr, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr),
                ONELA_ERR_INVALID_ARG);
      EXPECT_ST(onela_step(h, n, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr),
                ONELA_OK);
      onela_view view{};
      EXPECT_ST(onela_get_view(h, &view), ONELA_OK);
      EXPECT(view.t == t && view.n_beams == n && view.slots == B * L);
      b_prev = n;
    }
    EXPECT_ST(onela_get_status(h, nullptr), ONELA_OK);
    // capacity: a further step fails and changes nothing
    EXPECT_ST(onela_step(h, 1, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr),
              ONELA_ERR_CAPACITY);
    onela_view view{};
    EXPECT_ST(onela_get_view(h, &view), ONELA_OK);
    EXPECT(view.t == L);
    EXPECT_ST(onela_reset(h, nullptr), ONELA_OK);
    EXPECT_ST(onela_get_view(h, &view), ONELA_OK);
    EXPECT(view.t == 0 && view.n_beams == 1);
  }

  // a parent out of range raises the flag for this decode only
  if (L >= 2 && B >= 2) {
    for (int r = 0; r < R; ++r) parent[r] = 0;
    EXPECT_ST(onela_step(h, 1, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr), ONELA_OK);
    for (int r = 0; r < R * 2; ++r) parent[r] = 0;
    parent[1] = 5;  // the previous step had one beam
    EXPECT_ST(onela_step(h, 2, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr), ONELA_OK);
    EXPECT_ST(onela_get_status(h, nullptr), ONELA_ERR_BAD_PARENT);
    EXPECT_ST(onela_get_status(h, nullptr), ONELA_ERR_BAD_PARENT);  // sticky
    EXPECT_ST(onela_reset(h, nullptr), ONELA_OK);
    EXPECT_ST(onela_get_status(h, nullptr), ONELA_OK);
  }

  // a failed launch leaves the step count unchanged
  {
    for (int r = 0; r < R; ++r) parent[r] = 0;
    g_stub_fail_launch = 1;
    EXPECT_ST(onela_step(h, 1, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr),
              ONELA_ERR_DEVICE);
    onela_view view{};
    EXPECT_ST(onela_get_view(h, &view), ONELA_OK);
    EXPECT(view.t == 0);
    g_stub_fail_launch = 0;
  }

  // the regions the steps wrote (state, fragments, chains, plans, records) do not overlap
  EXPECT(stub_extents_disjoint());
  stub_extents_reset();

  // prefill installs a new context: t back to 0, flag cleared
  {
    const int N = 3;
    Buf pk((size_t)R * N * H * dk * 4), pv((size_t)R * N * H * dv * 4), pa((size_t)R * N * H * 4),
        pb((size_t)R * N * H * 4), out((size_t)R * H * dv * dk * 4);
    EXPECT_ST(onela_prefill(h, -1, pk.as<float>(), pv.as<float>(), pa.as<float>(), pb.as<float>(), nullptr, nullptr),
              ONELA_ERR_INVALID_ARG);
    EXPECT_ST(onela_prefill(h, N, nullptr, pv.as<float>(), pa.as<float>(), pb.as<float>(), nullptr, nullptr),
              ONELA_ERR_INVALID_ARG);
    EXPECT_ST(onela_prefill(h, N, pk.as<float>(), pv.as<float>(), pa.as<float>(), pb.as<float>(), out.as<float>(),
                            nullptr),
              ONELA_OK);
    EXPECT_ST(onela_prefill(h, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), ONELA_OK);
    onela_view view{};
    EXPECT_ST(onela_get_view(h, &view), ONELA_OK);
    EXPECT(view.t == 0);
    for (int r = 0; r < R; ++r) parent[r] = 0;
    EXPECT_ST(onela_step(h, 1, q.p, k.p, v.p, al.as<float>(), be.as<float>(), parent, o.as<float>(), nullptr), ONELA_OK);
  }

  // the handle belongs to its device
  g_stub_device = 1;
  EXPECT_ST(onela_reset(h, nullptr), ONELA_ERR_INVALID_ARG);
  g_stub_device = 0;
  EXPECT_ST(onela_destroy(h), ONELA_OK);
}

void run_select() {
  size_t bytes = 0;
  EXPECT_ST(onela_beam_select_scratch(0, 4, 8, 1, &bytes), ONELA_ERR_INVALID_ARG);
  EXPECT_ST(onela_beam_select_scratch(1, 4, 8, 33, &bytes), ONELA_ERR_INVALID_ARG);
  EXPECT_ST(onela_beam_select_scratch(1, 64, 64, 2049, &bytes), ONELA_ERR_UNSUPPORTED);
  EXPECT_ST(onela_beam_select_scratch(1, 4, 8, 3, nullptr), ONELA_ERR_INVALID_ARG);
  const int R = 3, n_prev = 100, n_cand = 300, K = 512;
  EXPECT_ST(onela_beam_select_scratch(R, n_prev, n_cand, K, &bytes), ONELA_OK);
  EXPECT(bytes > 0);
  Buf bs((size_t)R * n_prev * 4), lp((size_t)R * n_prev * n_cand * 4), scratch(bytes);
  Buf p((size_t)R * K * 4), t((size_t)R * K * 4), s((size_t)R * K * 4);
  EXPECT_ST(onela_beam_select(R, n_prev, n_cand, K, bs.as<float>(), lp.as<float>(), p.as<int32_t>(), t.as<int32_t>(),
                              s.as<float>(), scratch.p, bytes - 8, nullptr),
            ONELA_ERR_INVALID_ARG);
  EXPECT_ST(onela_beam_select(R, n_prev, n_cand, K, bs.as<float>(), lp.as<float>(), p.as<int32_t>(), nullptr,
                              s.as<float>(), scratch.p, bytes, nullptr),
            ONELA_ERR_INVALID_ARG);
  EXPECT_ST(onela_beam_select(R, n_prev, n_cand, K, bs.as<float>(), lp.as<float>(), p.as<int32_t>(), t.as<int32_t>(),
                              s.as<float>(), scratch.p, bytes, nullptr),
            ONELA_OK);
  EXPECT_ST(onela_beam_select_noalloc(R, n_prev, n_cand, K, bs.as<float>(), lp.as<float>(), p.as<int32_t>(),
                                      t.as<int32_t>(), s.as<float>(), nullptr),
            ONELA_OK);
  // 32 x 512 x 256 -> 2048 needs 16 MiB of scratch: more than the library holds
  Buf bs2((size_t)32 * 512 * 4), lp2((size_t)32 * 512 * 256 * 4), p2((size_t)32 * 2048 * 4), t2((size_t)32 * 2048 * 4),
      s2((size_t)32 * 2048 * 4);
  EXPECT_ST(onela_beam_select_noalloc(32, 512, 256, 2048, bs2.as<float>(), lp2.as<float>(), p2.as<int32_t>(),
                                      t2.as<int32_t>(), s2.as<float>(), nullptr),
            ONELA_ERR_CAPACITY);
  // fits without scratch
  EXPECT_ST(onela_beam_select_noalloc(1, 4, 8, 3, bs.as<float>(), lp.as<float>(), p.as<int32_t>(), t.as<int32_t>(),
                                      s.as<float>(), nullptr),
            ONELA_OK);
}

}  // namespace

int main() {
  // configurations the library rejects
  {
    size_t bytes = 0;
    onela_config bad[] = {make(0, 1, 16, 16, 4, 2, ONELA_F32, ONELA_MODE_REPLAY, 0, 0),
                          make(1, 1, 16, 257, 4, 2, ONELA_F32, ONELA_MODE_REPLAY, 0, 0),
                          make(1, 1, 16, 16, 4, 65, ONELA_F32, ONELA_MODE_REPLAY, 0, 0),
                          make(1, 1, 16, 16, 4, 2, 9, ONELA_MODE_REPLAY, 0, 0),
                          make(1, 1, 16, 16, 4, 2, ONELA_F32, 7, 0, 0),
                          make(1, 1, 16, 16, 4, 2, ONELA_F32, ONELA_MODE_REPLAY, 64, 0),
                          make(1, 1, 16, 16, 4, 2, ONELA_F32, ONELA_MODE_REPLAY, 0, 48),
                          make(1 << 20, 1 << 10, 256, 256, 1 << 20, 64, ONELA_F32, ONELA_MODE_REPLAY, 0, 0)};
    for (const onela_config& c : bad) EXPECT_ST(onela_workspace_size(&c, &bytes), ONELA_ERR_INVALID_ARG);
    EXPECT_ST(onela_workspace_size(nullptr, &bytes), ONELA_ERR_INVALID_ARG);
    onela_config ok = make(1, 1, 16, 16, 4, 2, ONELA_F32, ONELA_MODE_REPLAY, 0, 0);
    EXPECT_ST(onela_workspace_size(&ok, nullptr), ONELA_ERR_INVALID_ARG);
    EXPECT_ST(onela_destroy(nullptr), ONELA_ERR_INVALID_ARG);
    EXPECT_ST(onela_reset(nullptr, nullptr), ONELA_ERR_INVALID_ARG);
    EXPECT_ST(onela_get_view(nullptr, nullptr), ONELA_ERR_INVALID_ARG);
    for (int s = 0; s < 7; ++s) EXPECT(std::strncmp(onela_status_string((onela_status)s), "ONELA_", 6) == 0);
  }
  // every path of the host dispatch: fused bf16, both tiles; fp32 kernel; forced generic; materializing; FullState
  run_context(make(2, 3, 128, 128, 40, 4, ONELA_BF16, ONELA_MODE_REPLAY, 0, 0));
  run_context(make(1, 2, 128, 256, 33, 3, ONELA_BF16, ONELA_MODE_REPLAY, 0, 16));
  run_context(make(2, 1, 16, 24, 9, 3, ONELA_F32, ONELA_MODE_REPLAY, 0, 0));
  run_context(make(1, 2, 128, 64, 17, 2, ONELA_BF16, ONELA_MODE_REPLAY, ONELA_FLAG_FORCE_GENERIC, 0));
  run_context(make(2, 2, 32, 48, 6, 3, ONELA_F32, ONELA_MODE_REPLAY, ONELA_FLAG_MATERIALIZE, 0));
  run_context(make(1, 2, 16, 16, 5, 3, ONELA_BF16, ONELA_MODE_FULLSTATE, 0, 0));
  run_context(make(1, 1, 8, 8, 1, 1, ONELA_F32, ONELA_MODE_REPLAY, 0, 0));
  run_select();
  if (g_failures) std::fprintf(stderr, "%d checks failed\n", g_failures);
  else std::printf("host state machine: all checks passed\n");
  return g_failures ? 1 : 0;
}
