// Per-unit bookkeeping and state-tile helpers shared by the prefill kernels and the
// backward kernels: which (sequence, head) a workgroup serves, the S^T accumulator
// tiles of a value tile, and a value-row tile loaded ahead in accumulator layout.
#pragma once

#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {



template <typename Args>
__device__ __forceinline__ void unit_bounds(const Args& a, int unit, int& n_seq, int& h,
                                            int64_t& bos, int64_t& eos) {
  n_seq = unit / a.H;
  h = unit % a.H;
  if (a.cu_seqlens) {
    bos = a.cu_seqlens[n_seq];
    eos = a.cu_seqlens[n_seq + 1];
  } else {
    bos = static_cast<int64_t>(n_seq) * a.T;
    eos = bos + a.T;
  }
}

// Workgroup id -> (unit, role index) with W workgroups per unit.  With xcd_remap the
// W workgroups of a unit get ids congruent modulo 8 (the same XCD).
__device__ __forceinline__ void unit_role(int x, int W, int units, int xcd_remap, int& unit,
                                          int& role) {
  if (xcd_remap) {
    const int xcd = x & 7, y = x >> 3;
    unit = xcd * (units >> 3) + y / W;
    role = y % W;
  } else {
    unit = x / W;
    role = x % W;
  }
}

// S^T accumulator tiles of a value tile: wave w owns key blocks
// [w * KPW, (w + 1) * KPW) for every 16-row value block, KPW = DK / 64.
template <int DK, int BV>
struct StateTiles {
  static constexpr int NVB = BV / 16;
  static constexpr int KPW = DK / 64;
  static constexpr int NST = KPW * NVB;
  static __device__ __forceinline__ int kb(int wave, int s) { return wave * KPW + s / NVB; }
  static __device__ __forceinline__ int vb(int s) { return s % NVB; }
};

// Load the initial state tile (or zeros) into accumulators and its snapshot into LDS.
template <int DK, int BV, int LDK, typename TC, int NST>
__device__ __forceinline__ void load_state(f32x4 (&sacc)[NST], const float* s0, int64_t st_base,
                                           int v0, TC* sS, int wave, int lane) {
  using ST = StateTiles<DK, BV>;
  static_assert(NST == ST::NST, "state tile count");
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int s = 0; s < ST::NST; ++s) {
    const int kb = ST::kb(wave, s), vb = ST::vb(s);
    const int vrow = v0 + 16 * vb + lr, kcol = 16 * kb + 4 * lq;
    sacc[s] = s0 ? *reinterpret_cast<const f32x4*>(s0 + st_base + int64_t(vrow) * DK + kcol)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    store4(sS + (16 * vb + lr) * LDK + kcol, sacc[s]);
  }
}

template <int DK, int BV, int NST>
__device__ __forceinline__ void store_state(const f32x4 (&sacc)[NST], float* s1, int64_t st_base,
                                            int v0, int wave, int lane) {
  using ST = StateTiles<DK, BV>;
  static_assert(NST == ST::NST, "state tile count");
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int s = 0; s < ST::NST; ++s) {
    const int kb = ST::kb(wave, s), vb = ST::vb(s);
    const int vrow = v0 + 16 * vb + lr, kcol = 16 * kb + 4 * lq;
    *reinterpret_cast<f32x4*>(s1 + st_base + int64_t(vrow) * DK + kcol) = sacc[s];
  }
}

// Per-chunk buffers of the backward (chunk-start states, state gradients) are indexed
// by slot = chunk_slot_base(n, bos_n) + c for chunk c of sequence n.  Slots never
// collide: sequence n's last slot, floor(bos_n / 64) + n + ceil(len_n / 64) - 1, is
// below floor(bos_{n+1} / 64) + n + 1; chunk_slots_host() slots cover T_total packed rows.
__host__ __device__ inline int64_t chunk_slot_base(int n_seq, int64_t bos) {
  return bos / kChunk + n_seq;
}

// Per (chunk slot, head), in the backward's workspace, as 16-byte pieces: KD, Qg and -W
// [64][DK] bf16 (KD_r = k_r e^{G_n - G_r}, W = X diag(beta) Kg), M [64][64] bf16 (row r,
// column s: Qg_r . Ki_s for s <= r, else 0), e^{G_n} [DK] fp32.  Rows past a ragged
// chunk's end are zero.  The reverse chain reads them into LDS tiles with the row
// padding of kda_chunk.h.
template <int DK>
struct ChainTiles {
  static constexpr int PK = kChunk * DK / 8;       // pieces of a [64][DK] tile
  static constexpr int PC = kChunk * kChunk / 8;   // of a [64][64] tile
  static constexpr int PE = DK * 4 / 16;
  static constexpr int kPieces = 3 * PK + PC + PE;
  static constexpr size_t kBytes = size_t(kPieces) * 16;
  static constexpr size_t oW = size_t(2 * PK) * 16;   // byte offset of -W
  static constexpr size_t oM = size_t(3 * PK) * 16;   // byte offset of M
};

// LDS byte offset of piece p, given the byte offsets of the five tiles (KD, Qg, -W, M,
// e^{G_n}) with row strides DK + 8 and 64 + 8 (bf16).  The tile's offset is selected,
// not indexed: a run-time index into the table would put it in memory and cost a load
// (and a wait) per piece.
template <int DK>
__device__ __forceinline__ uint32_t piece_lds(const uint32_t (&off)[5], int p) {
  using TL = ChainTiles<DK>;
  constexpr int RK = DK / 8;
  if (p < 3 * TL::PK) {
    const int t = p / TL::PK, q = p % TL::PK;
    const uint32_t base = t == 0 ? off[0] : (t == 1 ? off[1] : off[2]);
    return base + ((q / RK) * (DK + 8) + 8 * (q % RK)) * 2;
  }
  p -= 3 * TL::PK;
  if (p < TL::PC) return off[3] + ((p / 8) * (kChunk + 8) + 8 * (p % 8)) * 2;
  return off[4] + 16 * (p - TL::PC);
}

// The state tile in accumulators as bf16 [d_v][d_k] rows at dst + base (four
// consecutive keys per lane: one 8-byte store per tile).
template <int DK, int BV, int NST>
__device__ __forceinline__ void store_state_bf16(const f32x4 (&sacc)[NST], bf16* dst, int64_t base,
                                                 int v0, int wave, int lane) {
  using ST = StateTiles<DK, BV>;
  static_assert(NST == ST::NST, "state tile count");
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int s = 0; s < ST::NST; ++s) {
    const int kb = ST::kb(wave, s), vb = ST::vb(s);
    const f32x4 x = sacc[s];
    *reinterpret_cast<bf16x4*>(dst + base + int64_t(v0 + 16 * vb + lr) * DK + 16 * kb + 4 * lq) =
        bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
               static_cast<bf16>(x[3])};
  }
}

// The value tile of one chunk in accumulator layout (row block = wave), loaded ahead
// as raw bits: bf16 in the low half of a 32-bit register, or fp32.
template <typename Tin, int NVB>
struct ValueRegs {
  uint32_t r[NVB][4];
  __device__ __forceinline__ void load(const Tin* v, int64_t c0, int n, int32_t H, int h,
                                       int32_t DV, int v0, int wave, int lane) {
    const Tin* vb0 = v + (c0 * H + h) * DV + v0;
    const uint32_t rowV = static_cast<uint32_t>(H) * DV;
    const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off =
            static_cast<uint32_t>(min(16 * wave + 4 * lq + i, n - 1)) * rowV + 16 * vb + lr;
        if constexpr (sizeof(Tin) == 2)
          r[vb][i] = *reinterpret_cast<const unsigned short*>(vb0 + off);
        else
          r[vb][i] = *reinterpret_cast<const uint32_t*>(vb0 + off);
      }
  }
  __device__ __forceinline__ float f32(int vb, int i) const {
    return sizeof(Tin) == 2 ? __uint_as_float(r[vb][i] << 16) : __uint_as_float(r[vb][i]);
  }
};

}  // namespace kda
