/*
 * probe.h -- measurement probes of the benchmark (libmsa_probe.so, built
 * beside libmsa.so but not part of it).  They are not on the MSA path: they
 * measure, on the GPU at hand, the two ceilings the path's kernels are read
 * against -- a streaming HBM read and the dense f16 MFMA issue rate -- so
 * that a kernel's fraction of the published peak can be set beside what the
 * chip actually sustains.
 *
 * Conventions as in msa.h: caller-owned device memory, asynchronous on
 * `stream`, argument errors returned before any HIP call, MSA_ERR_HIP when a
 * launch fails.
 */
#ifndef MSA_PROBE_H_
#define MSA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "../include/msa.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_PROBE_SINK_WORDS 4096

/* Reads `bytes` bytes of `buf` once: one workgroup per contiguous 32 KiB
 * slice, 16 bytes per lane per load, eight loads in flight per lane.
 *   buf    device, 16-byte aligned; bytes > 0 and a multiple of 16 (at most
 *          2^31 - 1 slices).
 *   sink   device, MSA_PROBE_SINK_WORDS uint32; written only when the XOR
 *          of the data a thread read equals a fixed magic value (so the
 *          reads cannot be optimised away). */
msa_status msa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Runs `iters` rounds of 16 independent 16x16x32 f16 MFMAs in every wave of
 * `workgroups` workgroups of 4 waves (no memory traffic in the loop):
 * workgroups * 4 * iters * 16 * 16384 flops.
 *   out    device, workgroups * 256 floats (one sum per thread).
 *   workgroups >= 1, iters >= 1. */
msa_status msa_probe_mfma_f16(float* out, int32_t workgroups, int32_t iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MSA_PROBE_H_ */
