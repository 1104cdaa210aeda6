/*
 * pagedattn_probe.h -- measurement entry point of libpagedattn.so (not a
 * step of the decode): a plain HBM read stream with no arithmetic beyond
 * folding the data, used to state the decode kernels' bandwidth as a
 * fraction of what the same access pattern reaches on the same GPU.
 */
#ifndef PAGEDATTN_PROBE_H
#define PAGEDATTN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads, for every page id pages[i] (0 <= i < num_pages), every run r
 * (0 <= r < runs_per_page) and each of base0 and base1 (base1 may be NULL),
 * the run_bytes bytes at
 *     base + pages[i] * page_stride + r * run_stride        (strides in BYTES)
 * with 16-byte nontemporal loads: the bytes a decode step gathers when the
 * page list holds its live blocks, a block's run is one kv head's keys (or
 * values), and runs_per_page is the number of kv heads. A contiguous read is
 * pages = 0, 1, 2, ... with page_stride = run_bytes.
 *
 * Every 16-byte piece read is XORed (as 4 dwords) into one of `workgroups`
 * * 256 per-thread 16-byte accumulators written to sink (uint32 [workgroups
 * * 256 * 4], caller-allocated), so the XOR of all sink entries is the XOR
 * of all bytes read, as 16-byte words.
 *
 * Device pointers; base0, base1, page_stride, run_stride and run_bytes must
 * be 16-byte aligned / multiples of 16, 16 <= run_bytes <= 8192, workgroups
 * >= 1, num_pages >= 0, runs_per_page >= 1. PA_EINVAL otherwise (pa_last_error
 * has the message). num_pages == 0 writes zero accumulators.
 */
int pa_read_probe(const void* base0, const void* base1, const int32_t* pages, int64_t num_pages,
                  int32_t runs_per_page, int64_t page_stride, int64_t run_stride, int32_t run_bytes,
                  uint32_t* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_PROBE_H */
