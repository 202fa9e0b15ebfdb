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

#ifdef __cplusplus
}
#endif

#endif
