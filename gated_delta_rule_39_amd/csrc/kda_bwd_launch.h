// Host-side launch interface of the backward kernels (kda_backward.hip) for the C ABI.
#pragma once

#include "kda_launch.h"

namespace kda {

// Arguments of the backward kernels (bf16 inputs; validated by the C ABI).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const void* dout;            // dL/do, layout of v
  const int32_t* cu_seqlens;
  const float* dfinal_state;   // dL/d(final state) or nullptr (zero)
  float* dinitial_state;       // dL/d(initial state) or nullptr (not written)
  void* dq;
  void* dk;
  void* dv;
  float* dg;                   // layout of g; unused without a decay
  float* dbeta;
  const void* states;          // bf16 [slot][H][d_v][d_k]: state at each chunk start
  void* dstates;               // bf16 [slot][H][d_v][d_k]: dL/d(state at each chunk end)
  void* tiles;                 // [slot][H] chunk tiles of the reverse chain
  int64_t T;
  int64_t slots;               // chunk_slots_host(T_total, N)
  int32_t H, DV, N, units;
  int32_t NV;                  // reverse chain: value tiles per unit
  int32_t xcd_remap;
  int32_t decay;
  int32_t flags;               // prologue flags of the forward call
  float scale;
};

hipError_t launch_backward_tiles(int dk, const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_chain(int dk, const BwdArgs& a, hipStream_t stream);
hipError_t launch_backward_grads(int dk, const BwdArgs& a, hipStream_t stream);
constexpr int kBwdChainBV = 16;   // value rows per reverse-chain workgroup
// Chunk slots of the backward's per-chunk buffers for T_total packed rows and N
// sequences (slot indexing: chunk_slot_base in kda_tiles.h).
inline int64_t chunk_slots_host(int64_t T_total, int32_t N) { return T_total / 64 + N + 1; }
// Bytes of one chunk's reverse-chain tiles (ChainTiles in kda_tiles.h): KD, Qg, -W
// [64][dk] and M [64][64] bf16, e^{G_n} [dk] fp32.
constexpr size_t chain_tile_bytes(int dk) {
  return size_t(3 * 64 * dk * 2 + 64 * 64 * 2 + dk * 4);
}

}  // namespace kda
