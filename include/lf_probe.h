/*
 * lf_probe.h - HBM bandwidth probes that sit beside the decode step.
 *
 * They are measuring tools, not part of the decode path: a plain streaming
 * copy (the reference traffic that hardware byte counters are scaled against),
 * a streaming read (the achievable read bandwidth of the device) and an empty
 * launch (the per-step floor).  Both
 * use the same 16-byte-per-lane coalesced access pattern as the decode kernel.
 * Device pointers, caller-owned; asynchronous on `stream` (hipStream_t as void*).
 */
#ifndef LF_PROBE_H_
#define LF_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "lf.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` (a multiple of 16, both pointers 16-byte aligned) from src to dst. */
lf_status lf_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Read `bytes` (a multiple of 16, 16-byte aligned) from src; writes one
 * uint32 per workgroup (an XOR of the data, so the loads cannot be elided)
 * into sink, which must hold at least lf_probe_read_sink_words() entries. */
lf_status lf_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
int32_t lf_probe_read_sink_words(void);

/* lf_probe_read over a grid of `n_blocks` workgroups (1 to
 * lf_probe_read_sink_words()) instead of the default: below a few hundred MB
 * per launch the fastest grid depends on the size (one workgroup per compute
 * unit reads 32-64 MB faster than the default grid), so a size-matched ceiling
 * takes the fastest of several.  sink receives n_blocks words.  Returns
 * LF_ERR_ARG for a grid outside that range. */
lf_status lf_probe_read_grid(const void* src, size_t bytes, int32_t n_blocks, uint32_t* sink, void* stream);

/* Launch `n_blocks` (>= 1) workgroups of 256 threads that do nothing.  Timed
 * in a graph of many such nodes it gives the launch floor a decode step of the
 * same grid pays before moving any byte. */
lf_status lf_probe_empty(int32_t n_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LF_PROBE_H_ */
