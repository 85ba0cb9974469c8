/*
 * pa_probe.h -- measurement probe of the paged-KV attention library: the
 * achievable HBM streaming-read bandwidth of the device.
 *
 * A decode step reads the request's whole KV cache and is bound by memory
 * bandwidth ("TensorRT-LLM, in depth" (aicassindra.com), section "First
 * principles: where the GPU memory goes"), so the context number for a decode
 * kernel's bandwidth is what a plain stream of the same loads reaches on the
 * same bytes.  This call reads a buffer once with the load form the decode
 * kernels use (16-byte non-temporal vector loads, whole 64-byte lines per
 * four lanes) and no other work, so its rate is the ceiling those loads can
 * reach; the published peak of the HBM stays the roofline.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at `src` (a DEVICE pointer, 16-byte aligned; bytes a
 * multiple of 16) once, in num_workgroups workgroups of 256 lanes
 * (1 .. 65536).  Workgroup w reads chunks w, w + num_workgroups, ... of
 * 256 * loads_in_flight consecutive 16-byte vectors, each lane holding
 * loads_in_flight (4, 8 or 16) loads in flight, then the bytes past the last
 * whole chunk.  Each wave writes the XOR of the words it read to
 * out[4 * workgroup + wave] (a DEVICE array of 4 * num_workgroups uint32,
 * caller-owned), so the loads are not removed; the values mean nothing else.
 * Queued on `stream`; allocates nothing.  Errors: PA_ERR_NULL_POINTER,
 * PA_ERR_MISALIGNED, PA_ERR_BAD_SHAPE, PA_ERR_UNSUPPORTED before any launch;
 * PA_ERR_HIP if the launch fails. */
pa_status pa_stream_read(const void *src, size_t bytes, uint32_t *out, int32_t num_workgroups,
                         int32_t loads_in_flight, void *stream);

/* The same for paged reads: read num_pages pages of page_bytes bytes (a positive
 * multiple of 1024) at base + page_offsets[i] (DEVICE pointers: base 16-byte aligned,
 * page_offsets an int64 array of byte offsets, each a multiple of 16, the pages inside
 * the caller's allocation), in list order.  The list is cut into equal contiguous
 * ranges, one per wave (4 waves per workgroup), each lane loading 16 bytes of every
 * kilobyte with pages_in_flight (2, 4 or 8) pages in flight -- the decode kernels'
 * pattern: a request's
 * blocks gathered through its table, one (block, kv head) page at a time ("How does
 * TensorRT-LLM work" (outcomeschool.com), section "The paged KV cache").  With the
 * pages a decode call visits, in its order, the rate is the achievable bandwidth of
 * that access pattern (pages of a few KB at random physical places).  out: 4 *
 * num_workgroups uint32, as for pa_stream_read.  Same errors. */
pa_status pa_gather_read(const void *base, const int64_t *page_offsets, int64_t num_pages, int32_t page_bytes,
                         uint32_t *out, int32_t num_workgroups, int32_t pages_in_flight, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
