/*
 * cl_probe.h -- measurement aids of the benchmark, exported by the same
 * library (libcompressed_linear.so).  They are not part of the forward: they
 * measure the two device limits a decode launch per layer meets, so that the
 * forward's rate can be read against what one kernel of a layer's size can
 * reach on the device at hand (the HBM roofline of the decode path).
 *
 * Return values: 0 on success, -1 for a bad argument, -4 for a launch failure,
 * -5 for a size beyond the launch grid.
 */
#ifndef CL_PROBE_H
#define CL_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * cl_probe_read -- one kernel that reads `bytes` (rounded down to 16) of the
 * device buffer `src` once with 16-byte nontemporal loads (eight in flight per
 * thread, 32 KiB per workgroup of 256 threads, 1 KiB contiguous per wavefront
 * load) and writes nothing but a guard word.
 *   src    device, 16-byte aligned, owned by the caller.
 *   sink   device, cl_probe_read_sink_words(bytes) uint32 words, caller owned.
 *   stream hipStream_t; asynchronous.
 */
int cl_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Words of `sink` that cl_probe_read needs for `bytes`. */
size_t cl_probe_read_sink_words(size_t bytes);

/* cl_probe_empty -- launch one empty kernel (one wavefront) on `stream`. */
int cl_probe_empty(void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CL_PROBE_H */
