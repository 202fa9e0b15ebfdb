// Host-side launchers of the gfx950 kernels (internal to libonela; the public ABI is include/onela.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace onela {

// Arguments of one decode step, shared by the replay kernels.
struct StepArgs {
  const void* q;          // [R][n][H][d_k] input dtype
  const void* k;          // [R][n][H][d_k]
  const void* v;          // [R][n][H][d_v]
  const float* alpha;     // [R][n][H]
  const float* beta;      // [R][n][H]
  float* o;               // [R][n][H][d_v]
  const float* sctx_t;    // [R][H][d_k][d_v]
  const uint16_t* sctx_frag;  // bf16 high/low MFMA fragments of S_ctx (fused kernel only)
  void* rec_k;            // [R][H][slots][d_k] input dtype
  float* rec_u;           // [R][H][slots][d_v]
  float* rec_alpha;       // [R][H][slots]
  const int32_t* chain;   // chain table after this step, [R][B_max][L_max] (read by the generic kernel)
  // ancestry inputs (the fused kernel derives chains itself and writes the new table)
  const int32_t* parent;      // [R][n]
  const int32_t* chain_prev;  // table after step t-1, NULL at t = 1
  int32_t* chain_out;         // table after step t
  int* flag;                  // set to `epoch` when a parent index is out of range
  int epoch;
  int b_prev;
  int R, H, d_k, d_v, n, B_max, L_max, slots, t;
};

hipError_t launch_ancestry(const int32_t* parent, const int32_t* chain_prev, int32_t* chain_out, int R, int n,
                           int b_prev, int B_max, int L_max, int t, int* flag, int epoch, hipStream_t s);
hipError_t launch_clear_flag(int* flag, hipStream_t s);
hipError_t launch_transpose_sctx(const float* S, float* ST, int RH, int d_v, int d_k, hipStream_t s);
hipError_t launch_split_frag(const float* ST, uint16_t* frag, int RH, int d_v, int d_k, hipStream_t s);
// GDN prefill from the zero state into sctx_t ([R][H][d_k][d_v]) and, if not NULL, sctx_out ([R][H][d_v][d_k]).
// scratch (scratch_bytes, 16-byte aligned, contents not preserved) serves the chunked MFMA form; with less than
// prefill_mfma_chunk_bytes(R, H) the row-parallel float32 kernel runs instead.
hipError_t launch_prefill(const float* k, const float* v, const float* alpha, const float* beta, int R, int H,
                          int N, int d_k, int d_v, float* sctx_t, float* sctx_out, void* scratch,
                          size_t scratch_bytes, hipStream_t s);
bool prefill_supported(int d_k, int d_v);
// chunked prefill on MFMA (d_k = 128, d_v in {16, 32, 64, 128, 256}); same outputs as launch_prefill.  The
// scratch holds the chunks' T for every (request, head): prefill_mfma_chunk_bytes(R, H) bytes per chunk; longer
// prompts run in segments of as many chunks as fit.
bool prefill_mfma_supported(int d_k, int d_v);
size_t prefill_mfma_chunk_bytes(int R, int H);
hipError_t launch_prefill_mfma(const float* k, const float* v, const float* alpha, const float* beta, int R, int H,
                               int N, int d_v, float* sctx_t, float* sctx_out, void* scratch, size_t scratch_bytes,
                               hipStream_t s);

hipError_t launch_step_generic(const StepArgs& a, bool bf16, hipStream_t s);
// Materializing replay (comparison path): dense parent state rebuilt per pair and step.
hipError_t launch_step_materialize(const StepArgs& a, bool bf16, hipStream_t s);

// Fused bf16-MFMA step (d_k of 64, 128 or 256, d_v % 32 == 0, 32 <= d_v <= 256, L_max <= 64), tiles of 16 or 32 beams.
// Steps t >= 2 first run the ancestry-plan kernel, which writes the chain table and per-tile plans into `plan`
// (fused_plan_bytes).  fused_prepare sets the kernel's LDS limit and returns its persistent grid size.
bool fused_supported(int d_k, int d_v, int L_max);
int fused_pick_tile(int d_k, int d_v, int L_max, int requested);
size_t fused_lds_bytes(int tile, int L_max, int d_k, int d_v);
size_t fused_plan_bytes(int R, int B_max, int L_max);
hipError_t fused_prepare(int tile, int d_k, int d_v, int L_max, int* grid);
hipError_t launch_step_fused(const StepArgs& a, int tile, void* plan, int grid, hipStream_t s);

// Beam selection: top n_beams of beam_score + logp per request, best first (beam_select.hip).
int beam_select_max_beams();
size_t beam_select_scratch_bytes(int R, long n, int n_beams);
hipError_t launch_beam_select(const float* beam_scores, const float* logp, int R, int n_prev, int n_cand,
                              int n_beams, int32_t* parent, int32_t* token, float* score, void* scratch,
                              hipStream_t s);
// The library-held scratch of the allocation-free entry point: its size, and its address on the current
// device (looked up on the first call per device).
size_t beam_select_static_max();
hipError_t beam_select_static_scratch(void** ptr);

hipError_t launch_fullstate(const StepArgs& a, bool bf16, const int32_t* parent, int b_prev, const float* fs_prev,
                            float* fs_next, hipStream_t s);

}  // namespace onela
