/* Bandwidth probe of libonela_probe.so: plain streaming kernels that give the bench the HBM rate a simple
 * kernel reaches for a given read/write mix on this GPU (context for the decode step's roofline fraction; not
 * part of the decode library).
 *
 * onela_probe_stream enqueues one kernel of 256-thread workgroups on `stream`: with grid = 0, one element per
 * thread (ceil(n / 256) workgroups); with grid > 0, that many workgroups in a grid-stride loop.  Every access is a
 * 16-byte vector load or store and n counts 16-byte elements:
 *   mode 0 read    src holds 2n elements, all read; with grid > 0 sink (grid x 256 floats) receives per-thread
 *                  sums (with grid = 0 sink must still be a valid device pointer; it is almost never written)
 *   mode 1 mix     src holds 2n elements, all read; dst holds 3n elements, all written (2 : 3 bytes)
 *   mode 2 copy    src and dst hold n elements; dst = src
 *   mode 3 write   dst holds n elements, all written with a constant
 * Buffers are device memory owned by the caller, 16-byte aligned.  Returns 0 when enqueued, 1 for a bad
 * argument (nothing enqueued), 2 when the launch failed. */
#ifndef ONELA_PROBE_H
#define ONELA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int onela_probe_stream(const void* src, void* dst, size_t n, int mode, float* sink, int grid, void* stream);

/* onela_probe_step_traffic enqueues the first decode step's memory traffic without its arithmetic: one 256-thread
 * workgroup per (request, head, tile of 32 beams), no LDS, no barriers.  It reads the tile's rows of k and q (bf16,
 * d_k = 128) and v (bf16, d_v), laid out [R][B][H][d] as onela_step takes them, and alpha and beta ([R][B][H]
 * float32); the first tile of each (request, head) also reads 128 * d_v * 4 bytes of sctx at offset
 * (request * H + head) * 128 * d_v * 4.  It writes o ([R][B][H][d_v] float32), and rows of u (d_v float32), of
 * the key (d_k bf16) and the alpha at slot b of arenas laid out [R * H][slots].  The values written are folded
 * from those read (the probe measures bandwidth; they mean nothing).  B a multiple of 32, d_v a multiple of 32
 * up to 256, slots >= B; buffers are device memory owned by the caller, 16-byte aligned.  Returns 0 when
 * enqueued, 1 for a bad argument (nothing enqueued), 2 when the launch failed. */
int onela_probe_step_traffic(const void* k, const void* q, const void* v, const float* alpha, const float* beta,
                             const void* sctx, void* o, void* u, void* rec_k, float* rec_alpha, int R, int B, int H,
                             int d_v, int slots, void* stream);

#ifdef __cplusplus
}
#endif

#endif
