/*
 * hyb_probe.h - HBM bandwidth probe of libhyb.so: a measurement aid, not part of the attention
 * step. It streams a device buffer with plain kernels so that the attention kernels' achieved
 * bytes per second can be set against the rate this GPU's memory delivers in practice, beside
 * the published peak. Same status codes, error string and stream rules as include/hyb.h.
 *
 * hyb_probe - one launch of `variant` with n_workgroups workgroups of 256 threads:
 *   HYB_PROBE_READ        each workgroup reads its contiguous share of src[0, bytes), `unroll`
 *                         16-byte loads per thread in flight (unroll 4, 8 or 16)
 *   HYB_PROBE_READ_DYN    workgroups take chunks of page_bytes from *counter (atomic add) until
 *                         the buffer is exhausted; *counter must be 0 at launch and holds the
 *                         number of grabs afterwards (the caller clears it between launches)
 *   HYB_PROBE_READ_LDS    as READ, through direct global -> LDS loads (4 KB stages per wave,
 *                         three in flight); unroll is ignored
 *   HYB_PROBE_READ_PAGES  the n_pages pages src + pages[j] * page_bytes (page_bytes each), in list
 *                         order, split evenly over the workgroups (a shuffled paged pool)
 *   HYB_PROBE_COPY        dst[0, bytes) <- src[0, bytes)
 *   src, dst   device memory, 16-byte aligned; dst only for COPY (else may be NULL)
 *   bytes      a multiple of hyb_probe_granule(variant, unroll) (READ_PAGES: unused)
 *   page_bytes READ_DYN: grab size, READ_PAGES: page size (a multiple of the granule)
 *   pages      int32 [n_pages] (device), each page inside src - the caller's to keep in range
 *   trace      optional uint64 [n_workgroups][4] (device): per workgroup its XCC (die) id, start
 *              and end ticks of the 100 MHz real-time counter, and the bytes it moved
 * ------------------------------------------------------------------------------------------ */
#ifndef HYB_PROBE_H
#define HYB_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hyb_probe_variant {
  HYB_PROBE_READ = 0,
  HYB_PROBE_READ_DYN = 1,
  HYB_PROBE_READ_LDS = 2,
  HYB_PROBE_READ_PAGES = 3,
  HYB_PROBE_COPY = 4
} hyb_probe_variant;

uint64_t hyb_probe_granule(int32_t variant, int32_t unroll);
int32_t hyb_probe(int32_t variant, int32_t unroll, int32_t n_workgroups, const void* src,
                  void* dst, uint64_t bytes, uint32_t* counter, const int32_t* pages,
                  int32_t n_pages, int64_t page_bytes, uint64_t* trace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HYB_PROBE_H */
