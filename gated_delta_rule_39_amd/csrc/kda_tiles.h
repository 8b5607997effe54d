// Per-unit bookkeeping and state-tile helpers shared by the prefill kernels and the
// backward kernels: which (sequence, head) a workgroup serves, the S^T accumulator
// tiles of a value tile, and a value-row tile loaded ahead in accumulator layout.
#pragma once

#include "kda_chunk.h"
#include "kda_launch.h"
#include "kda_wy.h"

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

// Per (chunk slot, head), in the backward's workspace: KD (KD_r = k_r e^{G_n - G_r}),
// Qg^T and -W^T (W = X diag(beta) Kg) as bf16 MFMA operand fragments of 1 KiB (64 lanes
// x 16 bytes, lane-major), M [64][64] bf16 row-major (row r, column s: Qg_r . Ki_s for
// s <= r, else 0), then e^{G_n} [DK] fp32.  Fragments of KD, block tb * (DK / 32) + s:
// lane l holds row 16 tb + l % 16, keys 32 s + 8 (l / 16) .. +7.  Qg^T and -W^T, block
// 2 kb + u: lane l holds key 16 kb + l % 16, tokens 32 u + 8 (l / 16) .. +7.  Rows past a
// ragged chunk's end are zero.  The reverse chain loads each wave's fragments straight
// into registers, one contiguous 1 KiB per load.
template <int DK>
struct ChainTiles {
  static constexpr int PK = kChunk * DK / 8;       // 16-byte pieces of a 64 x DK tile
  static constexpr int PC = kChunk * kChunk / 8;   // of a [64][64] tile
  static constexpr int PE = DK * 4 / 16;
  static constexpr int kPieces = 3 * PK + PC + PE;
  static constexpr size_t kBytes = size_t(kPieces) * 16;
  static constexpr size_t oKD = 0, oQT = size_t(PK) * 16, oWT = size_t(2 * PK) * 16;
  static constexpr size_t oM = size_t(3 * PK) * 16, oE = size_t(3 * PK + PC) * 16;
};

// Writers of a chunk's tiles from a workgroup's LDS (non-temporal stores: the tiles are
// read only by a later kernel).  KD fragments from a row-major
// [64][DK] bf16 tile (each element multiplied by e^{G_n} of its key when scale_egn).
template <int DK>
__device__ __forceinline__ void store_kd_frags(unsigned char* dst, const bf16* sKD, int ld,
                                               const float* egn, bool scale_egn, int wave,
                                               int lane) {
  using TL = ChainTiles<DK>;
  constexpr int NKS = DK / 32;
  for (int f = wave; f < 4 * NKS; f += 4) {
    const int tb = f / NKS, s = f % NKS;
    bf16x8 x = frag_rows<Mfma<bf16>>(sKD, ld, 16 * tb, 32 * s, lane);
    if (scale_egn) {
      const int k0 = 32 * s + 8 * (lane >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = static_cast<bf16>(static_cast<float>(x[e]) * egn[k0 + e]);
    }
    __builtin_nontemporal_store(x, reinterpret_cast<bf16x8*>(dst + TL::oKD + 1024 * size_t(f) +
                                                             16 * lane));
  }
}

// The transpose of a row-major [64][DK] bf16 LDS tile as fragments at dst: block
// 2 kb + u, lane l: column 16 kb + l % 16, rows 32 u + 8 (l / 16) .. +7 (one transposing
// read per fragment).
template <int DK>
__device__ __forceinline__ void store_tr_frags(unsigned char* dst, const bf16* src, int ld,
                                               int wave, int lane) {
  for (int f = wave; f < 2 * (DK / 16); f += 4) {
    const int kb = f >> 1, u = f & 1;
    __builtin_nontemporal_store(frag_tr(src, ld, 32 * u, 16 * kb, lane),
                                reinterpret_cast<bf16x8*>(dst + 1024 * size_t(f) + 16 * lane));
  }
}

// e^{G_n} of the chunk (fp32 [DK]) at its place in the tiles.
template <int DK>
__device__ __forceinline__ void store_egn(unsigned char* dst, const float* egn, int tid) {
  using TL = ChainTiles<DK>;
  if (tid < TL::PE)
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(egn + 4 * tid),
                                reinterpret_cast<f32x4*>(dst + TL::oE + 16 * size_t(tid)));
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
