/*
 * kda_noalloc.h -- the allocation-free variant of kda_prefill_ex (libkda.so), for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Conventions and status codes as
 * kda.h, plus KDA_ERR_SCRATCH.
 */
#ifndef KDA_NOALLOC_H
#define KDA_NOALLOC_H

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The call needs more workspace than the library's fixed scratch. */
enum { KDA_ERR_SCRATCH = 7 };

/* Bytes of the per-device scratch array behind kda_prefill_noalloc. */
#define KDA_NOALLOC_SCRATCH_BYTES (96u << 20)

/*
 * kda_prefill_noalloc -- kda_prefill_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace; the producer/consumer kernel's
 * workspace is a library-owned device array of KDA_NOALLOC_SCRATCH_BYTES (96 MiB) per
 * device, held from the first call on that device until the process ends.  The call
 * makes no allocation of any kind.  Returns KDA_ERR_SCRATCH, launching nothing, when
 * the call needs more (kda_prefill_workspace_bytes() above the limit).  With the
 * default plans on a 256-CU device every call fits: at d_k = d_v = 128 the units
 * share at most 32 lanes whatever their number (about 72 MiB), and one unit per lane
 * needs at most about 84 MiB (d_k = 128, d_v = 64, 42 units).  When the fused kernel applies (fp32, or no
 * producer/consumer plan) it runs without scratch.  Every call on one
 * device shares that device's array: calls that overlap in time on one device (other
 * streams, other threads) race and give undefined results; calls ordered on one
 * stream are safe.  An aborted hand-off is visible only in the outputs (NaN, as for
 * kda_prefill); the abort words live in the library's array.
 */
int kda_prefill_noalloc(int dtype, int decay, int flags,
                        const void* q, const void* k, const void* v,
                        const float* g, const float* beta,
                        const int32_t* cu_seqlens,
                        int32_t N, int32_t B, int64_t T, int32_t H, int32_t d_k, int32_t d_v,
                        float scale,
                        const float* initial_state, float* final_state,
                        void* o, hipStream_t stream);

/* KDA_NOALLOC_SCRATCH_BYTES, as built into the library. */
size_t kda_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_NOALLOC_H */
