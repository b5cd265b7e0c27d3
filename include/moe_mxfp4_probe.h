/*
 * moe_mxfp4_probe.h -- measurement helpers of the MXFP4 MoE library.
 *
 * Not part of the layer.  They give the HBM roofline that the expert
 * kernels are reported against: the pages put a 1T MoE's decode time in
 * weight I/O (yifor-blog digest, memory-bandwidth section), so the achieved
 * fraction of the bandwidth a plain streaming read reaches is the number
 * that matters; and a copy of known size calibrates the hardware counters
 * (FETCH_SIZE / WRITE_SIZE) used to measure HBM traffic.
 *
 * Device pointers, caller-owned, 16-byte aligned; `bytes` a multiple of 16.
 * Work is enqueued on `stream` (a hipStream_t, NULL = null stream).
 * Returns 0, or a negative status of include/moe_mxfp4.h (MOE_E_NULL,
 * MOE_E_SHAPE, MOE_E_ALIGN, MOE_E_HIP).
 */
#ifndef MOE_MXFP4_PROBE_H
#define MOE_MXFP4_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` from src with 128-bit nontemporal loads across the whole
 * GPU, each workgroup streaming contiguous 256 KB ranges (the expert
 * kernels' access pattern); one uint32 per thread (a fold of what it read)
 * goes to sink, which must hold moe_probe_sink_words() words. */
int moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* The same read with ordinary loads, which allocate in L2 and the Infinity
 * Cache: reading more than those hold evicts them without leaving dirty
 * lines to write back (a cold step's setup). */
int moe_probe_read_cached(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Words the sink of moe_probe_stream_read / moe_probe_read_cached must hold. */
int64_t moe_probe_sink_words(void);

/* Copy `bytes` from src to dst with 128-bit loads and stores. */
int moe_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_PROBE_H */
