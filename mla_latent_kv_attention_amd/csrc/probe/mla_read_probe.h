/*
 * mla_read_probe.h -- measurement helper of the benchmark, built as its own library
 * (libmla_read_probe.so); not part of the attention C-ABI in include/mla.h.
 *
 * mla_hbm_read_probe reads `bytes` of device memory once and keeps nothing: each of
 * `grid` work-groups of 256 threads streams one contiguous share with 16-byte loads
 * and writes one word per thread to `sink`.  Timed by the caller, it gives the rate at
 * which the device delivers that many bytes to a kernel that does nothing else: the
 * practical ceiling of an HBM-bound kernel that must read them once, next to the
 * published peak.
 *
 * src     device, 16-byte aligned, `bytes` readable bytes (bytes % 16 == 0).
 * sink    device, grid * 256 uint32 (overwritten; contents meaningless).
 * grid    1 .. 65536 work-groups.
 * stream  hipStream_t to launch on.
 * Returns 0, -1 for a null pointer, a misaligned src or size, or a grid out of range
 * (before any launch), or -4 if the launch failed.
 */
#ifndef MLA_READ_PROBE_H_
#define MLA_READ_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mla_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_READ_PROBE_H_ */
