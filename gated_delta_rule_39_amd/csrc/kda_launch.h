// Host-side launch interface between the C ABI (kda_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Prologue flags: inputs given as raw projections.  kNormK: k is L2-normalised per
// (token, head) over d_k, k / sqrt(sum k^2 + kNormEps); kBetaLogit: beta = sigmoid(beta);
// kGateLogit: the gate input a gives the retention alpha = sigmoid(a) (g = log alpha).
constexpr int kNormK = 1, kBetaLogit = 2, kGateLogit = 4;
constexpr float kNormEps = 1e-6f;

// Arguments of both prefill kernels (validated by the C ABI).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;
  const float* initial_state;
  float* final_state;
  void* o;
  unsigned char* workspace;   // producer/consumer kernel only
  int64_t T;
  int32_t H, DV, units;
  int32_t NV;                 // fused kernel: value tiles per unit
  int32_t NC, NP, R;          // producer/consumer kernel: consumers, producers, ring slots
  int32_t lanes;              // producer/consumer kernel: workgroup sets (lanes)
  // lane l processes units lane_units[lane_off[l] .. lane_off[l + 1]) one after another
  // (planned on the device, in the workspace); nullptr: lane l is unit l
  const int32_t* lane_off;
  const int32_t* lane_units;
  int32_t xcd_remap;          // units % 8 == 0: keep a unit's workgroups on one XCD
  int32_t decay;              // 0: g per key channel, 1: one g per (token, head), 2: none
  int32_t flags;              // prologue flags (kda_device.h: kNormK, kBetaLogit, kGateLogit)
  float scale;
  void* chunk_states;         // STATES instantiations: bf16 state at every chunk start
  void* chunk_tiles;          // STATES producer/consumer kernel: each chunk's factor tiles
};

// Backward: the forward sweep that writes the chunk-start states (fused kernel, bf16,
// a.workspace = states), then the reverse chain and the chunk-parallel gradients.
hipError_t launch_prefill_states(int dk, int bv, const PrefillArgs& a, hipStream_t stream);
// The same from the producer/consumer kernel (d_k = d_v = 128, two consumers of 64 value
// columns; a.o may be nullptr); a.workspace as for launch_prefill_coop.
hipError_t launch_prefill_coop_states(const PrefillArgs& a, hipStream_t stream);
// dtype: 0 = fp32, 1 = bf16; dk, dv in {64, 128}.
// decay: 0 = g per key channel [units, dk], 1 = one g per unit [units], 2 = none.
hipError_t launch_decode(int dtype, int decay, int flags, int dk, int dv, const void* q,
                         const void* k, const void* v, const float* g, const float* beta,
                         float* state, void* o, int32_t units, float scale, hipStream_t stream);
// Fused prefill: bv in {16, 32, 64}, bv <= prefill_max_bv(dtype, dk), a.NV = DV / bv.
hipError_t launch_prefill(int dtype, int dk, int bv, const PrefillArgs& a, hipStream_t stream);
int prefill_max_bv(int dtype, int dk);
// Producer/consumer prefill (bf16): a.workspace holds prefill_coop_workspace_bytes bytes;
// a.DV / (4 * a.NC) in {16, 32}.
hipError_t launch_prefill_coop(int dk, const PrefillArgs& a, hipStream_t stream);
// lanes sets of workgroups; plan: the units are spread over the lanes by a device plan
// (lanes < units), else lane l is unit l (lanes == units).
size_t prefill_coop_workspace_bytes(int dk, int dv, int lanes, int units, int R, bool plan);
// The argument checks of kda_prefill_ex (kda_api.cpp), no HIP call: a kda.h status,
// and *launch = false when there is nothing to do.
int prefill_args_status(int dtype, int decay, int flags, const void* q, const void* k,
                        const void* v, const float* g, const float* beta,
                        const int32_t* cu_seqlens, int32_t N, int32_t B, int64_t T, int32_t H,
                        int32_t d_k, int32_t d_v, const float* final_state, const void* o,
                        bool* launch);

}  // namespace kda
