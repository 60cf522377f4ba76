/*
 * mpb_probe.h -- C ABI of libmpb_probe.so, a measurement helper that the
 * benchmark uses beside libmpb.so.  It is not part of the attention path:
 * nothing in libmpb.so calls it and it reads or writes no plan or tensor.
 */
#ifndef MPB_PROBE_H_
#define MPB_PROBE_H_

#include <stdint.h>

#include "mpb.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 MFMA throughput probe for gfx950: launches `workgroups`
 * workgroups of four wavefronts, each wavefront issuing iters * 8
 * independent v_mfma_f32_32x32x16_bf16 (32768 flops each; the instruction
 * the attention kernels use) on register operands, and writes one float per
 * thread to `out` (device, workgroups * 256 floats).  Flops per launch:
 * workgroups * 4 * iters * 8 * 32768; the caller times the launch on
 * `stream` to measure the MFMA rate the device sustains at the clock it runs
 * under that load.  MPB_ERR_INVALID_ARGUMENT for a non-positive count or a
 * NULL out, MPB_ERR_DEVICE if the launch fails.  Enqueue only. */
mpb_status mpb_mfma_probe(int32_t workgroups, int32_t iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MPB_PROBE_H_ */
