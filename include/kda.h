/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * The operation (per independent unit = one sequence, one head): a state S with
 * d_v rows and d_k columns maps keys to values.  For each token t, with
 * alpha_t = exp(g_t) per key channel:
 *   decay    S~  = S_{t-1} Diag(alpha_t)          (column j scaled by alpha_t[j])
 *   predict  p   = S~ k_t
 *   error    e   = beta_t (v_t - p)
 *   correct  S_t = S~ + e k_t^T
 *   read     o_t = S_t (scale q_t)
 * Source: "Kimi Delta Attention: The Linear Attention Behind Kimi K2 and Qwen3"
 * (elsolitario.org), section "How Kimi Delta Attention works step by step"
 * (listing and flowchart); scale defaults to d_k^{-1/2} there.  Chunked prefill
 * and in-place one-token decode follow "Kimi Delta Attention Technical Deep Dive"
 * (mohalkarushikesh.github.io), "Systems and implementation tradeoffs"
 * ("Training", "Decoding", "Kernel design": one state layout for both paths).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP device memory of the current
 *    device), row-major and contiguous in the layouts stated.  The caller owns
 *    every buffer; the library allocates nothing and keeps no state except a
 *    per-device cached compute-unit count.
 *  - Calls enqueue work on `stream` and return at once; nothing synchronises with
 *    the host.  A device fault surfaces at the caller's next synchronisation.
 *  - Every argument is validated before any HIP call.  Status codes are below;
 *    nothing throws across the ABI.
 *  - Unchecked device-side preconditions: keys L2-normalised; g <= 0; beta in
 *    [0, 2]; cu_seqlens non-decreasing with cu[0] = 0 and cu[N] = B*T; and a bound on
 *    the decay within a 64-token chunk (chunks start at each sequence's first token),
 *    as a sum of |g| per key channel: on the bf16 producer/consumer prefill, below
 *    about 85 over every aligned 16 tokens of a chunk (chunks in which some 8 tokens
 *    decay by more than e^-10 are factored per 16-token block); on the fused prefill
 *    kernel (fp32, and bf16 shapes without a producer/consumer plan) and in the
 *    backward, below about 80 over the whole chunk.  Outside these the numerics are
 *    defined but not guaranteed; NaN propagates.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

/* dtype of q, k, v and o.  g, beta and all states are always fp32. */
enum { KDA_F32 = 0, KDA_BF16 = 1 };

/*
 * How the state decays at each token (the `_ex` entry points; the plain ones are
 * KDA_DECAY_CHANNEL).  The three members of the family share the decay -> predict ->
 * correct -> read cycle and differ in the decay ("Kimi Delta Attention: The Linear
 * Attention Behind Kimi K2 and Qwen3", "From quadratic attention to fixed state: a
 * brief history" and "DeltaNet, Gated DeltaNet, and KDA: comparison table"):
 *   KDA_DECAY_CHANNEL  KDA: per key channel, g is [.., H, d_k]
 *   KDA_DECAY_HEAD     Gated DeltaNet: one scalar per (token, head), g is [.., H]
 *   KDA_DECAY_NONE     DeltaNet: no decay, g is not read (may be NULL)
 */
enum { KDA_DECAY_CHANNEL = 0, KDA_DECAY_HEAD = 1, KDA_DECAY_NONE = 2 };

/*
 * Prologue flags (the `_ex` entry points; 0 = inputs as the plain entry points take
 * them).  They fuse the step just before the recurrence, which turns a layer's raw
 * projections into its inputs: unit keys (the delta rule assumes them: "Kimi Delta
 * Attention: The Linear Attention Behind Kimi K2 and Qwen3", warning in "How Kimi
 * Delta Attention works step by step" and FAQ "Why does DeltaNet need keys to be
 * normalized?"), a sigmoid-like retention and a positive write strength ("Kimi
 * Delta Attention Technical Deep Dive", "From attention to recurrent state").
 *   KDA_PRO_NORM_K      k is raw: each (token, head) row is replaced by
 *                       k / sqrt(sum_j k_j^2 + 1e-6) before use (the prefill
 *                       rounds the unit key of bf16 inputs to bf16 again, its
 *                       MFMA operand type; the decode step keeps it in fp32)
 *   KDA_PRO_BETA_LOGIT  beta holds logits: beta <- 1 / (1 + exp(-beta))
 *   KDA_PRO_GATE_LOGIT  g holds retention logits a: alpha = 1 / (1 + exp(-a))
 *                       (instead of alpha = exp(g)); ignored with KDA_DECAY_NONE
 * q is never normalised (it is scaled by `scale`).
 */
enum { KDA_PRO_NORM_K = 1, KDA_PRO_BETA_LOGIT = 2, KDA_PRO_GATE_LOGIT = 4 };
enum {
  KDA_OK = 0,
  KDA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                          */
  KDA_ERR_BAD_SHAPE = 2,    /* negative or inconsistent sizes                      */
  KDA_ERR_UNSUPPORTED = 3,  /* d_k or d_v not in {64, 128}, unknown decay kind or
                               prologue flag                                        */
  KDA_ERR_BAD_DTYPE = 4,    /* dtype not KDA_F32 / KDA_BF16                         */
  KDA_ERR_HIP = 5,          /* kernel launch failed (hipGetLastError)              */
  KDA_ERR_WORKSPACE = 6     /* workspace NULL or smaller than the call needs       */
};

/* Returns KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_string(int status);

/*
 * kda_prefill -- chunked (64-token chunks) forward over N sequences.
 *
 * Layout: token rows are packed as [B, T, H, d]: element (row r, head h,
 * channel j) is at ((r * H + h) * d + j).
 *   q, k : [B, T, H, d_k]  dtype      v, o : [B, T, H, d_v]  dtype
 *   g    : [B, T, H, d_k]  fp32 (log alpha)
 *   beta : [B, T, H]       fp32
 *   cu_seqlens : [N + 1] int32 on the device, or NULL.  With NULL, N must equal B
 *     and sequence n is batch row n (rows n*T .. n*T+T-1).  Otherwise B must be 1
 *     and sequence n is rows cu[n] .. cu[n+1]-1 of the T packed rows; empty
 *     sequences are allowed.
 *   initial_state : [N, H, d_v, d_k] fp32, or NULL for zeros.
 *   final_state   : [N, H, d_v, d_k] fp32, or NULL (not written).  It may alias
 *     initial_state exactly (each state tile is read before it is written).
 *   o : written for every token row that belongs to a sequence.
 * N = 0 or T = 0 is a no-op returning KDA_OK (nothing launched).
 * scale: query scale (the pages use d_k^{-1/2}).
 * workspace / workspace_bytes: optional device scratch.  With bf16 inputs, when
 *   kda_prefill_workspace_bytes() is nonzero and the workspace holds at least that
 *   many bytes, the producer/consumer kernel runs: per (sequence, head), producer
 *   workgroups compute each chunk's d_v-independent tiles once and hand them to the
 *   value-tile workgroups through a ring in the workspace.  Otherwise (NULL, too
 *   small, fp32) the fused kernel runs, in which every value tile recomputes them.
 *   The library owns the workspace's contents during the call (no initialisation
 *   needed) except its second int32; calls that share one workspace must be ordered
 *   on one stream.  Abort report: after such a call completes, the workspace's
 *   first int32 is 0; nonzero means a cross-workgroup hand-off wait timed out and
 *   the call stopped early.  Every output element of a (sequence, head) that did
 *   not complete is then NaN (o rows, final state), so an aborted call never leaves
 *   stale values that look valid.  The second int32 is sticky: an aborted call sets
 *   it to 1 and no call clears it, so a caller that zeroes it once can check many
 *   calls with one read.
 *   Launch: the producer/consumer grid is a cooperative launch, whose workgroups are
 *   all resident at once.  With the environment variable KDA_COOP_LAUNCH=plain it is
 *   an ordinary dispatch of the same grid when the device can hold all of it at
 *   once (about 20 us less per call); the hand-off waits are bounded either way, so
 *   a grid that were not fully resident (another such grid in flight on another
 *   stream) aborts as above rather than hanging.
 */
int kda_prefill(int dtype,
                const void* q, const void* k, const void* v,
                const float* g, const float* beta,
                const int32_t* cu_seqlens,
                int32_t N, int32_t B, int64_t T, int32_t H, int32_t d_k, int32_t d_v,
                float scale,
                const float* initial_state, float* final_state,
                void* o,
                void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * kda_prefill_ex -- kda_prefill with the decay kind and the prologue flags as
 * arguments.  With KDA_DECAY_HEAD, g is [B, T, H] fp32 (one log-decay, or retention
 * logit, per token row and head); with KDA_DECAY_NONE, g is not read and may be
 * NULL.  Everything else is as kda_prefill.
 */
int kda_prefill_ex(int dtype, int decay, int flags,
                   const void* q, const void* k, const void* v,
                   const float* g, const float* beta,
                   const int32_t* cu_seqlens,
                   int32_t N, int32_t B, int64_t T, int32_t H, int32_t d_k, int32_t d_v,
                   float scale,
                   const float* initial_state, float* final_state,
                   void* o,
                   void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* Workspace bytes that select the producer/consumer prefill for these sizes on the
 * current device (0: not applicable, the fused kernel runs).  Host-only apart from a
 * cached device-attribute query. */
size_t kda_prefill_workspace_bytes(int dtype, int32_t N, int64_t T_total, int32_t H,
                                   int32_t d_k, int32_t d_v);

/* Geometry of the producer/consumer prefill on the current device: value-tile
 * workgroups (consumers), producer workgroups per lane and ring slots; all zero when
 * it does not apply.  For a call with per-channel decay (kda_prefill); a call without
 * decay and without prologue flags runs one producer fewer where six would fit (the
 * workspace size is the same).  Output pointers may be NULL. */
int kda_prefill_coop_plan(int dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                          int32_t* consumers, int32_t* producers, int32_t* ring_slots);

/* Lanes of the producer/consumer prefill (0: it does not apply).  A lane is one set
 * of consumer and producer workgroups working through a stream of chunks.  With as
 * many lanes as (sequence, head) units, lane i is unit i.  With d_k = d_v = 128 and
 * more units than the device has room for lanes of seven workgroups (N <= 256,
 * N * H <= 8192), a plan made on the device from cu_seqlens at each call spreads the
 * units over fewer lanes, longest sequences first, each to the lane with the least
 * work so far; a lane then processes its units one after another, each with its own
 * boundary state carried from chunk to chunk ("Kimi Delta Attention Technical Deep
 * Dive", "Systems and implementation tradeoffs" -> "Training").
 * Host-only apart from a cached device-attribute query. */
int kda_prefill_coop_lanes(int dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v);

/*
 * Launch geometry of the fused prefill kernel on the current device: the number of
 * d_v tiles each (sequence, head) is split into (rows of S never mix, so the
 * tiles run independently) and the resulting workgroup count.  Either output
 * pointer may be NULL.  Host-only apart from a cached device-attribute query.
 */
int kda_prefill_plan(int dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                     int32_t* v_tiles, int32_t* workgroups);

/*
 * kda_decode_step -- one token per (sequence, head); the state is advanced IN
 * PLACE ("Decoding": one state update and one query-state product per token,
 * cost independent of the context length).
 *   q, k : [N, H, d_k] dtype     v, o : [N, H, d_v] dtype
 *   g    : [N, H, d_k] fp32      beta : [N, H] fp32
 *   state: [N, H, d_v, d_k] fp32, read and overwritten.
 * N = 0 is a no-op returning KDA_OK.
 */
int kda_decode_step(int dtype,
                    const void* q, const void* k, const void* v,
                    const float* g, const float* beta,
                    float* state, void* o,
                    int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                    float scale, hipStream_t stream);

/*
 * kda_decode_step_ex -- kda_decode_step with the decay kind and the prologue flags
 * as arguments.  With KDA_DECAY_HEAD, g is [N, H] fp32; with KDA_DECAY_NONE, g is
 * not read and may be NULL.  Everything else is as kda_decode_step.
 */
int kda_decode_step_ex(int dtype, int decay, int flags,
                       const void* q, const void* k, const void* v,
                       const float* g, const float* beta,
                       float* state, void* o,
                       int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                       float scale, hipStream_t stream);

/*
 * kda_backward -- gradients of kda_prefill_ex (training).  The pages tie the chunkwise
 * form to training ("Kimi Delta Attention Technical Deep Dive", "Systems and
 * implementation tradeoffs" -> "Training") and give no gradient formulas; this is the
 * exact gradient of the recurrence of "Kimi Delta Attention: The Linear Attention
 * Behind Kimi K2 and Qwen3", "How Kimi Delta Attention works step by step", for a
 * loss whose gradients with respect to o and to the final state are given.
 *   dtype: KDA_BF16 only (KDA_F32 returns KDA_ERR_UNSUPPORTED).
 *   Inputs decay, flags, q, k, v, g, beta, cu_seqlens, N, B, T, H, d_k, d_v, scale,
 *     initial_state: exactly as passed to the forward call (kda_prefill_ex).  With
 *     prologue flags the gradients are with respect to the raw inputs: dk through the
 *     key normalisation, dbeta through the sigmoid, dg through g = log sigmoid(a).
 *   dout : [B, T, H, d_v] bf16, dL/do.
 *   dfinal_state : [N, H, d_v, d_k] fp32, dL/d(final state), or NULL (zero).
 *   Outputs (caller-allocated, written for every token row of a sequence):
 *     dq, dk : [B, T, H, d_k] bf16      dv : [B, T, H, d_v] bf16
 *     dg     : layout of g, fp32 (not read or written with KDA_DECAY_NONE; may be NULL)
 *     dbeta  : [B, T, H] fp32
 *     dinitial_state : [N, H, d_v, d_k] fp32, dL/d(initial state), or NULL (not written).
 *   workspace: device memory of at least kda_backward_workspace_bytes() bytes (else
 *     KDA_ERR_WORKSPACE); it receives the state at every chunk start, the state
 *     gradient at every chunk end (bf16) and every chunk's factor tiles, and is owned
 *     by the library during the call.
 *     With d_k = d_v = 128 and the producer/consumer plan of kda_prefill_coop_plan()
 *     (two consumers), the forward sweep that recomputes the chunk states runs on that
 *     kernel and the workspace starts with its ring: after the call, a nonzero first
 *     int32 means a hand-off wait timed out and the outputs are invalid (the chunk
 *     states of the units that did not complete are NaN, and so are their
 *     gradients); the second int32 is the sticky abort word, as for kda_prefill.
 * N = 0 is a no-op returning KDA_OK.  The keys must be unit rows as for the forward.
 */
int kda_backward(int dtype, int decay, int flags,
                 const void* q, const void* k, const void* v,
                 const float* g, const float* beta,
                 const int32_t* cu_seqlens,
                 int32_t N, int32_t B, int64_t T, int32_t H, int32_t d_k, int32_t d_v,
                 float scale, const float* initial_state,
                 const void* dout, const float* dfinal_state,
                 void* dq, void* dk, void* dv, float* dg, float* dbeta,
                 float* dinitial_state,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Workspace bytes kda_backward needs, with S = (T_total / 64 + N + 1) * H chunk slots:
 * 2 * S * d_v * d_k * 2 for the chunk states and state gradients (bf16), plus
 * S * (388 d_k + 8192) for each chunk's factor tiles (bf16 KD, Qg, W, M; fp32 e^{G_n}),
 * plus the producer/consumer ring when that forward sweep applies (0 for unsupported
 * arguments).  Host-only apart from a cached device-attribute query. */
size_t kda_backward_workspace_bytes(int dtype, int32_t N, int64_t T_total, int32_t H,
                                    int32_t d_k, int32_t d_v);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
