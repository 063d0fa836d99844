/*
 * pa_probe.h -- measurement helper of the decode library on MI355X (gfx950):
 * C ABI of libpa_probe.so, a library of its own that only the benchmark loads.
 *
 * pa_read_probe: the achievable HBM read rate, against which the decode
 * kernels' rates are read (the decode is a bandwidth-bound gather,
 * "PagedAttention: Virtual Memory for the KV Cache", section 13).  Reads every
 * byte of `buf` (device, `bytes` a multiple of 4096) once: wave w of the
 * `workgroups` workgroups of 256 threads reads the 4 KiB pieces w, w + W, ...
 * (W waves), four pieces of 16-byte loads in flight, and one word per
 * workgroup goes to `sink` (device, uint32 [workgroups]).  `nontemporal` 1
 * marks the loads non-temporal (the cache policy the decode kernels stream
 * the KV pool with), 0 leaves the default policy.  Asynchronous on `stream`
 * (a hipStream_t as void*); time it with events.  Returns 0, or 1 (bytes not
 * a multiple of 4096, workgroups outside 1..65535, nontemporal not 0 or 1,
 * NULL buffers) before any launch, or 7 when the runtime refused the launch.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, int workgroups, int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
