/*
 * kda_probe.h -- measurement probes exported by libkda.so beside the KDA entry points
 * of kda.h.  They compute nothing of the method: they measure what one MI355X
 * (gfx950) delivers, so that the benchmark can report its kernels against measured
 * peaks as well as the published ones (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).
 *
 * Conventions as kda.h: device pointers, asynchronous on `stream`, validation before
 * any HIP call, status codes of kda.h (KDA_OK, KDA_ERR_NULL_ARG, KDA_ERR_BAD_SHAPE,
 * KDA_ERR_HIP).  The caller owns every buffer and times the call (HIP events).
 */
#ifndef KDA_PROBE_H
#define KDA_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HBM stream: copy `bytes` (a multiple of 16, at least 16) from src to dst with
 * 16-byte non-temporal loads and stores; moves 2 * bytes.  src and dst must not
 * overlap and must be 16-byte aligned. */
int kda_probe_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* HBM read stream: read `bytes` (a multiple of 16, at least 16) of src with 16-byte
 * non-temporal loads; each workgroup writes one 32-bit word of a fold of what it read
 * to sink[workgroup] (sink holds kda_probe_read_sink_words() words). */
int kda_probe_hbm_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
int32_t kda_probe_read_sink_words(void);

/* Dense bf16 MFMA loop: `workgroups` workgroups of four waves; each wave issues
 * iters x 8 independent v_mfma_f32_16x16x32_bf16 (16384 flop each) and writes one
 * float to sink[workgroup] (sink holds `workgroups` floats) only if its result is a
 * given improbable value, so the work is not optimised away.
 * Flops = workgroups * 4 * iters * 8 * 16384. */
int kda_probe_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PROBE_H */
