/*
 * sdpa_probe.h - C ABI of libsdpa_probe.so, a measurement helper that is not
 * part of the attention method: it measures the bf16 matrix-core throughput
 * this GPU sustains at the clock it actually runs, so a benchmark can report
 * its kernels against that ceiling next to the published dense peak.
 *
 * Ownership and errors: `out` is a DEVICE buffer owned by the caller, holding
 * at least n_workgroups * 256 floats (the probe writes one value per thread so
 * the work cannot be optimised away; the values carry no meaning). Work is
 * enqueued on `stream`; the call returns after the enqueue and keeps no state.
 */
#ifndef SDPA_PROBE_H
#define SDPA_PROBE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch n_workgroups workgroups of 4 waves; each wave issues iters x 8
 * v_mfma_f32_32x32x16_bf16 in two independent accumulator chains on register
 * operands. Returns 0, -1 for a null `out` or a non-positive count, -4 if the
 * launch failed. */
int sdpa_probe_mfma_bf16(float* out, int32_t n_workgroups, int32_t iters, hipStream_t stream);

/* FLOP that one sdpa_probe_mfma_bf16 call with these counts performs. */
double sdpa_probe_mfma_bf16_flop(int32_t n_workgroups, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_PROBE_H */
