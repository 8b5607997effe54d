// The KDA chunk step in WY form, split between producer and consumer workgroups
// (gfx950, bf16 operands, fp32 accumulation).
//
// With X = (I + A)^{-1} and the chunk factors of kda_chunk.h, the state step of one
// chunk (n <= 64 rows) is
//   E     = U - W S^T              U = X diag(beta) V,   W = X diag(beta) Kg
//   O     = Qg S^T + M E
//   S'^T  = D S^T + KD^T E         D = Diag(e^{G_n}),   KD_{r,j} = k_{r,j} e^{G_{n,j} - G_{r,j}}
// (substitute E = X diag(beta)(V - Kg S^T) and S' = (S + E^T Ki) D of kda_chunk.h).
// W, U, Qg, KD^T, M and e^{G_n} depend on the chunk's inputs only.  A producer
// computes them once per (unit, chunk) and publishes them into a ring slot; a
// consumer owning a block of value columns keeps its part of S^T in MFMA
// accumulators and runs the chain E -> S' -> E ... with operands from registers:
// the recurrent state stays in registers and the prediction, error, gate and write
// of each token are fused into the chunk step, as the kernel-design notes of "Kimi
// Delta Attention Technical Deep Dive" (mohalkarushikesh.github.io, "Systems and
// implementation tradeoffs" -> "Kernel design") ask.
//
// Permuted-K fragments.  A 16x16 accumulator holds D[4g + i][l % 16] in lane l
// (g = l / 16, i = 0..3).  Two accumulators of consecutive 16-row blocks 2j, 2j+1
// packed into eight bf16 per lane form a 16x32 MFMA operand fragment whose lane l
// covers row (or column) l % 16 and K indices
//   32j + 4g + e        (e = 0..3,  from block 2j)
//   32j + 16 + 4g + e-4 (e = 4..7,  from block 2j+1).
// The MFMA sums over K, so any K order works as long as both operands use it.  All
// published fragments use this order; then every accumulator a consumer produces
// (S^T, E) is directly the next product's operand, as the A operand (rows = value
// column) or the B operand (columns = value column): no LDS round trip in the chain.
// The producer forms W and M transposed (W^T = Kg^T (X diag(beta))^T, M^T = Ki Qg^T)
// so that their accumulators are the published fragments too.
#pragma once

#include "kda_chunk.h"

namespace kda {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two accumulators of row blocks 2j, 2j+1 -> one permuted-K operand fragment.
__device__ __forceinline__ bf16x8 pack_frag(f32x4 lo, f32x4 hi) {
  return bf16x8{static_cast<bf16>(lo[0]), static_cast<bf16>(lo[1]), static_cast<bf16>(lo[2]),
                static_cast<bf16>(lo[3]), static_cast<bf16>(hi[0]), static_cast<bf16>(hi[1]),
                static_cast<bf16>(hi[2]), static_cast<bf16>(hi[3])};
}

// The same fragment from a row-major bf16 LDS array: row row0 + l % 16, K from k0.
__device__ __forceinline__ bf16x8 frag_perm(const bf16* base, int ld, int row0, int k0, int lane) {
  const bf16* p = base + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane j
// supplies the address of four consecutive bf16 and lane i receives element i % 4 of
// the vectors addressed by lanes 4e + i / 4, e = 0..3.  With lane j addressing row
// R + j / 4, column n0 + 4 (j % 4) of a row-major array, lane i receives column n0 + i
// of rows R .. R + 3.
__device__ __forceinline__ bf16x4 read_tr4(const bf16* base, int ld, int row, int col) {
  typedef __bf16 v4bf16 __attribute__((__vector_size__(4 * sizeof(__bf16))));
  const auto p = (__attribute__((address_space(3))) v4bf16*)(base + row * ld + col);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p));
}

// MFMA operand fragment of a row-major K x N bf16 LDS array (K = row index): lane l
// covers column n0 + l % 16 and K rows k0 + 8 (l / 16) .. +7 (the order frag_rows
// uses for an N x K array).
__device__ __forceinline__ bf16x8 frag_tr(const bf16* base, int ld, int k0, int n0, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const bf16x4 a = read_tr4(base, ld, k0 + 8 * g + (j >> 2), n0 + 4 * (j & 3));
  const bf16x4 b = read_tr4(base, ld, k0 + 8 * g + 4 + (j >> 2), n0 + 4 * (j & 3));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The same in the permuted K order: rows k0 + 4 (l / 16) .. +3, then k0 + 16 + 4 (l / 16)
// .. +3 (k0 = 32 j).
__device__ __forceinline__ bf16x8 frag_tr_perm(const bf16* base, int ld, int k0, int n0, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const bf16x4 a = read_tr4(base, ld, k0 + 4 * g + (j >> 2), n0 + 4 * (j & 3));
  const bf16x4 b = read_tr4(base, ld, k0 + 16 + 4 * g + (j >> 2), n0 + 4 * (j & 3));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// A fragment times per-K factors: s[0..7] for the K order of frag_rows (eight
// consecutive K), or s[0..3], s[16..19] for frag_perm.
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 f, f32x4 lo, f32x4 hi) {
  return bf16x8{static_cast<bf16>(static_cast<float>(f[0]) * lo[0]),
                static_cast<bf16>(static_cast<float>(f[1]) * lo[1]),
                static_cast<bf16>(static_cast<float>(f[2]) * lo[2]),
                static_cast<bf16>(static_cast<float>(f[3]) * lo[3]),
                static_cast<bf16>(static_cast<float>(f[4]) * hi[0]),
                static_cast<bf16>(static_cast<float>(f[5]) * hi[1]),
                static_cast<bf16>(static_cast<float>(f[6]) * hi[2]),
                static_cast<bf16>(static_cast<float>(f[7]) * hi[3])};
}
__device__ __forceinline__ bf16x8 scale_rows8(bf16x8 f, const float* s) {
  return scale_frag(f, *reinterpret_cast<const f32x4*>(s), *reinterpret_cast<const f32x4*>(s + 4));
}
__device__ __forceinline__ bf16x8 scale_perm8(bf16x8 f, const float* s) {
  return scale_frag(f, *reinterpret_cast<const f32x4*>(s), *reinterpret_cast<const f32x4*>(s + 16));
}
__device__ __forceinline__ bf16x8 scale_all(bf16x8 f, float x) {
  const f32x4 v = f32x4{x, x, x, x};
  return scale_frag(f, v, v);
}

__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += A B for 16x16 fp32 blocks on the fp32 MFMA, in the permuted K order: step s
// sums k = 4 (l / 16) + s, so lane l supplies A[l % 16][4 (l / 16) + s] (one 16-byte
// read of a row-major A) and b[s] = B[4 (l / 16) + s][l % 16] -- exactly the values a
// 16x16 accumulator holds in lane l.  A product of products then needs no LDS round
// trip.
__device__ __forceinline__ f32x4 mm16p(f32x4 acc, const float* A, int lda, f32x4 b, int lane) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(A + (lane & 15) * lda + 4 * (lane >> 4));
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}
// The b operand of mm16p from a row-major fp32 LDS block.
__device__ __forceinline__ f32x4 acc_layout(const float* B, int ldb, int lane) {
  const float* p = B + 4 * (lane >> 4) * ldb + (lane & 15);
  return f32x4{p[0], p[ldb], p[2 * ldb], p[3 * ldb]};
}

// ---- ring slot ---------------------------------------------------------------------
// One chunk's published operands.  Every fragment block is the 16 bytes each of 64
// lanes holds (1 KiB, lane-major), so a block is copied with one 16-byte-per-lane
// load and read with one conflict-free ds_read_b128.
//   W   (tb, j)  tb < 4 token blocks, j < DK/32          rows = token
//   Q   (tb, j)  the same for Qg
//   KD  (kb, t)  kb < DK/16 key blocks, t < 2           rows = key channel
//   M   (tb, t)  t = 0 for tb < 4, then t = 1 for tb = 2, 3 (the others are zero),
//                block index tb for t = 0, 2 + tb for t = 1
//   egn DK fp32 (in a 1 KiB block)
//   U   (tb, p)  p < DV/32: the 16x16 accumulator tiles of value blocks 2p and 2p + 1
//                rounded to bf16, lane l holding its four values of each (16 bytes)
// The consumer copies [0, kStage) -- fragments, egn and padding -- into LDS.
template <int DK, int DV>
struct WySlot {
  static constexpr int KS = DK / 32;
  static constexpr size_t kFrag = 1024;
  static constexpr int nW = 4 * KS;
  static constexpr int nKD = 2 * (DK / 16);
  static constexpr int nM = 6;
  static constexpr size_t oW = 0;
  static constexpr size_t oQ = oW + nW * kFrag;
  static constexpr size_t oKD = oQ + nW * kFrag;
  static constexpr size_t oM = oKD + nKD * kFrag;
  static constexpr size_t oEgn = oM + nM * kFrag;
  // staged part padded to a multiple of 4 blocks: each consumer wave copies the same
  // number of blocks
  static constexpr int nStage = static_cast<int>((oEgn / kFrag + 1 + 3) / 4 * 4);
  static constexpr size_t kStage = size_t(nStage) * kFrag;
  static constexpr size_t oU = kStage;
  static constexpr int NVB = DV / 16;
  static constexpr size_t kBytes = oU + 4 * (NVB / 2) * kFrag;
  static_assert(DK * 4 <= static_cast<int>(kFrag), "egn block");
};

// ---- producer ----------------------------------------------------------------------
template <int DK, int DV>
struct WyProducerLayout {
  static constexpr int LDK = DK + 8;        // bf16 [64][DK] rows, 16-byte pad
  static constexpr int LDV = DV + 8;        // bf16 [64][DV] rows
  static constexpr int LDC = kChunk + 8;    // bf16 [*][64] rows
  static constexpr int LDF = kChunk + 4;    // fp32 [64][64]
  static constexpr int CG = DK / 4, RG = kThreads / CG;
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t tK = size_t(kChunk) * LDK * 2;
  static constexpr size_t oKg = 0;
  static constexpr size_t oQg = al(oKg + tK);
  static constexpr size_t oKi = al(oQg + tK);
  static constexpr size_t oKD = al(oKi + tK);                          // [64][LDK]
  static constexpr size_t oV = al(oKD + tK);                           // [64][LDV]
  static constexpr size_t oTm = al(oV + size_t(kChunk) * LDV * 2);     // X diag(beta), [64][LDC]
  static constexpr size_t oA = al(oTm + size_t(kChunk) * LDC * 2);     // fp32 [64][LDF]
  static constexpr size_t oX = al(oA + size_t(kChunk) * LDF * 4);      // fp32 [64][LDF]
  static constexpr size_t scrTot = size_t(RG) * DK * 4;
  static constexpr size_t scrY = size_t(4) * 16 * 17 * 4;
  static constexpr size_t oScr = al(oX + size_t(kChunk) * LDF * 4);
  static constexpr size_t oBeta = al(oScr + (scrTot > scrY ? scrTot : scrY));
  static constexpr size_t oEgn = al(oBeta + kChunk * 4);
  // strong-decay chunks: block-pair factors [7][DK] and block-start decays [4][DK]
  static constexpr size_t oPair = al(oEgn + DK * 4);
  static constexpr size_t oEc = al(oPair + size_t(7) * DK * 4);
  static constexpr size_t oFlag = al(oEc + size_t(4) * DK * 4);
  static constexpr size_t kBytes = al(oFlag + 16);
};

// Device-scope (SC1) buffer accesses for ring slots: a store is acknowledged once it
// is visible device-wide and a load reads the device-coherent copy, so the hand-off
// needs no cache write-back or invalidate.
constexpr int kDeviceScope = 16;
// Non-temporal (NT) bit of a buffer instruction's cache policy.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(unsigned char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void ring_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16x8 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ void ring_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kDeviceScope);
}
// One 1 KiB block: 64 lanes x 16 bytes from the ring at off + 16 * lane into LDS at
// dst + 16 * lane (dst wave-uniform).  Completion is counted by vmcnt, not lgkmcnt,
// and the compiler does not order later LDS reads after it: wait explicitly.
__device__ __forceinline__ void ring_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void* dst,
                                            int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(dst), 16, off + 16 * lane, 0,
      0, kDeviceScope);
}

template <int DK, int DV>
struct WyProducer {
  using L = WyProducerLayout<DK, DV>;
  using SL = WySlot<DK, DV>;
  using M = Mfma<bf16>;
  static constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDF = L::LDF;
  static constexpr int CG = DK / 4, RG = kThreads / CG, RPG = kChunk / RG;
  // v rows are only copied to LDS: eight channels per thread (16-byte loads)
  static constexpr int CGV = DV / 8, RGV = kThreads / CGV, RPGV = kChunk / RGV;
  static constexpr int KS = DK / 32;

  bf16 *sKg, *sQg, *sKi, *sKD, *sV, *sTm;
  float *sA, *sX, *sScr, *sBeta, *sEgn, *sPair, *sEc;
  int* sStrong;
  // this chunk takes the strong-decay factorization (wave-uniform; set by factors())
  bool strong;
  const bf16 *q, *k, *v;
  const float *g, *beta;
  int32_t H, h;
  uint32_t rowK, rowV;
  int tid, lane, wave, rg, j0, rgv, jv0;
  float scale;
  f32x4 gr[RPG];
  bf16x4 kr[RPG], qr[RPG];
  bf16x8 kp[RPG / 2], qp[RPG / 2], vr[RPGV];   // k, q as loaded (pairs of rows), v rows
  float br;
  int32_t flags;   // prologue flags (kNormK, kBetaLogit, kGateLogit)
  // slot stores: plain when the unit's workgroups share one L2, else device-scope
  bool local;
  __device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16x8 v) const {
    if (local)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
    else
      ring_store16(r, off, v);
  }
  __device__ __forceinline__ void st4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) const {
    if (local)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
    else
      ring_store4(r, off, v);
  }

  __device__ __forceinline__ void init(unsigned char* smem, const bf16* q_, const bf16* k_,
                                       const bf16* v_, const float* g_, const float* beta_,
                                       int32_t H_, int32_t h_, float scale_, int tid_, int wave_,
                                       int32_t flags_) {
    flags = flags_;
    sKg = reinterpret_cast<bf16*>(smem + L::oKg);
    sQg = reinterpret_cast<bf16*>(smem + L::oQg);
    sKi = reinterpret_cast<bf16*>(smem + L::oKi);
    sKD = reinterpret_cast<bf16*>(smem + L::oKD);
    sV = reinterpret_cast<bf16*>(smem + L::oV);
    sTm = reinterpret_cast<bf16*>(smem + L::oTm);
    sA = reinterpret_cast<float*>(smem + L::oA);
    sX = reinterpret_cast<float*>(smem + L::oX);
    sScr = reinterpret_cast<float*>(smem + L::oScr);
    sBeta = reinterpret_cast<float*>(smem + L::oBeta);
    sEgn = reinterpret_cast<float*>(smem + L::oEgn);
    sPair = reinterpret_cast<float*>(smem + L::oPair);
    sEc = reinterpret_cast<float*>(smem + L::oEc);
    sStrong = reinterpret_cast<int*>(smem + L::oFlag) + 2;
    strong = false;
    q = q_;
    k = k_;
    v = v_;
    g = g_;
    beta = beta_;
    H = H_;
    h = h_;
    rowK = static_cast<uint32_t>(H_) * DK;
    rowV = static_cast<uint32_t>(H_) * DV;
    scale = scale_;
    tid = tid_;
    lane = tid_ & 63;
    wave = wave_;
    rg = tid_ / CG;
    j0 = 4 * (tid_ % CG);
    rgv = tid_ / CGV;
    jv0 = 8 * (tid_ % CGV);
    br = 0.f;
    local = false;
    // no chunk tag is negative (a barrier follows before the first chunk)
    if (tid == 0) *sStrong = -1;
    // the strictly upper part of X diag(beta) is never written
    for (int i = tid; i < kChunk * LDC; i += kThreads) sTm[i] = static_cast<bf16>(0.f);
  }

  // Rows c0 .. c0+n-1 (n >= 1) of the inputs into registers.  The loads form one list
  // (g rows, k rows, q rows, v rows, beta) of which the caller issues slices between the
  // phases of a chunk, so that the per-CU memory pipeline never holds more than one
  // slice of misses; rows past the end re-read the last valid row (masked at use).
  // Streaming (non-temporal) loads: the inputs are read once.  BUF: buffer loads at
  // 32-bit byte offsets from the chunk's first row (fewer address instructions than
  // 64-bit flat addresses; the plan keeps 64 rows within 2 GiB).  Measured: 1 % faster
  // in the forward kernel, 3 % slower in the sweep that also writes states and tiles,
  // which keeps flat loads.
  // The list, in order: g rows [0, kSK), k [kSK, kSQ), q [kSQ, kSV), v [kSV, kSB), beta.
  // k and q take 16-byte loads: the two lanes of a pair (l, l ^ 1) share a row group and
  // the eight channels j0 & ~7 .. +7; lane l loads rows 2m + (l & 1) of them, and
  // unpack_pairs() swaps the halves within the pair.
  static constexpr int kSK = RPG, kSQ = RPG + RPG / 2, kSV = 2 * RPG, kSB = 2 * RPG + RPGV;
  static constexpr int kLoads = kSB + 1;
  template <int DECAY, int I0, int I1, bool BUF = true>
  __device__ __forceinline__ void load_slice(int64_t c0, int n, int h) {
    const int64_t rk = (c0 * H + h) * DK;
    auto rsrc = [](const void* p) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rsk = rsrc(k + rk), rsq = rsrc(q + rk),
                                 rsv = rsrc(v + (c0 * H + h) * DV);
#pragma unroll
    for (int e = I0; e < I1; ++e) {
      if (e < kSK) {
        const int i = e;
        const uint32_t off = static_cast<uint32_t>(min(rg * RPG + i, n - 1)) * rowK + j0;
        // g per key channel; with one g per (row, head), lane l loads row l's and
        // factors() hands the rows to the threads that use them; no g: zeros
        if constexpr (DECAY == 0) {
          if constexpr (BUF)
            gr[i] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(g + rk), off * 4, 0, kNonTemporal));
          else
            gr[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + rk + off));
        } else if constexpr (DECAY == 1) {
          if (i == 0) gr[0][0] = g[(c0 + min(lane, n - 1)) * H + h];
        } else {
          gr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      } else if (e < kSV) {
        const bool isk = e < kSQ;
        const int m = isk ? e - kSK : e - kSQ;
        const uint32_t off =
            static_cast<uint32_t>(min(rg * RPG + 2 * m + (lane & 1), n - 1)) * rowK + (j0 & ~7);
        bf16x8 x;
        if constexpr (BUF)
          x = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                             isk ? rsk : rsq, off * 2, 0, kNonTemporal));
        else
          x = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>((isk ? k : q) + rk + off));
        if (isk)
          kp[m] = x;
        else
          qp[m] = x;
      } else if (e < kSB) {
        const int i = e - kSV;
        const uint32_t ov = static_cast<uint32_t>(min(rgv * RPGV + i, n - 1)) * rowV + jv0;
        vr[i] = BUF ? __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rsv, ov * 2, 0, kNonTemporal))
                    : __builtin_nontemporal_load(
                          reinterpret_cast<const bf16x8*>(v + (c0 * H + h) * DV + ov));
      } else {
        br = __builtin_nontemporal_load(beta + (c0 + min(lane, n - 1)) * H + h);
      }
    }
  }
  // k and q rows in the per-thread layout (row rg RPG + i, channels j0 .. j0 + 3) from
  // the pair loads: a lane keeps its own half of the rows it loaded and takes its half of
  // its partner's rows with one DPP swap (quad_perm [1, 0, 3, 2]).
  __device__ __forceinline__ void unpack_pairs() {
    const bool odd = (lane & 1) != 0;
    auto swap = [](uint32_t x) {
      return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), 0xb1, 0xf, 0xf, false));
    };
    auto unpack = [&](const bf16x8(&p)[RPG / 2], bf16x4(&r)[RPG]) {
#pragma unroll
      for (int m = 0; m < RPG / 2; ++m) {
        const u32x4 x = __builtin_bit_cast(u32x4, p[m]);
        // the partner's channels of the row this lane loaded
        const uint32_t r0 = swap(odd ? x[0] : x[2]), r1 = swap(odd ? x[1] : x[3]);
        r[2 * m] = __builtin_bit_cast(bf16x4, u32x2{odd ? r0 : x[0], odd ? r1 : x[1]});
        r[2 * m + 1] = __builtin_bit_cast(bf16x4, u32x2{odd ? x[2] : r0, odd ? x[3] : r1});
      }
    };
    unpack(kp, kr);
    unpack(qp, qr);
  }
  template <int DECAY, bool BUF = true>
  __device__ __forceinline__ void load(int64_t c0, int n, int h) {
    load_slice<DECAY, 0, kLoads, BUF>(c0, n, h);
  }

  // Kg, Qg, Ki, KD, V (row-major), beta and e^{G_n} of the loaded chunk into LDS.  The
  // input registers are free afterwards.  No closing barrier.
  // Raw keys to unit keys: row norms over the CG threads of a row group, then the
  // normalised key rounded to bf16 again (what a caller-side normalisation hands over).
  __device__ __forceinline__ void normalise_keys() {
    float ss[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const f32x4 k4 = widen(kr[i]);
      ss[i] = dot4(k4, k4);
    }
#pragma unroll
    for (int i = 0; i < RPG; ++i) ss[i] = row_sum<CG>(ss[i]);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const f32x4 k4 = widen(kr[i]) * __builtin_amdgcn_rsqf(ss[i] + kNormEps);
      kr[i] = bf16x4{static_cast<bf16>(k4[0]), static_cast<bf16>(k4[1]),
                     static_cast<bf16>(k4[2]), static_cast<bf16>(k4[3])};
    }
  }

  // The strong-decay tiles of factors() (QSCALE as there): Kg, Qg from the start of
  // the row's 16-row block, Ki to its end, KD to the chunk end; the block-pair factors
  // [1 / Bd_0 .. 1 / Bd_3, Bd_1, Bd_2, Bd_1 Bd_2] (Bd_a: decay over block a) and the
  // block-start decays Ec_a = Bd_0 .. Bd_{a-1}.
  template <bool QSCALE>
  __device__ __forceinline__ void strong_factors(const f32x4 (&tots)[RG], f32x4 cs, int n) {
    constexpr int GPB = 16 / RPG;   // row groups per 16-row block
    const f32x4 one = f32x4{1.f, 1.f, 1.f, 1.f};
    f32x4 bp = one, bs = one;       // this block's groups before / after this one
#pragma unroll
    for (int r2 = 0; r2 < RG; ++r2)
      if (r2 / GPB == rg / GPB) {
        if (r2 < rg) bp *= tots[r2];
        if (r2 > rg) bs *= tots[r2];
      }
    f32x4 kf[RPG];
    f32x4 run = bp;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      run *= gr[i];
      kf[i] = widen(kr[i]);
      f32x4 q4 = widen(qr[i]);
      if constexpr (QSCALE) q4 *= scale;
      store4(sKg + (rg * RPG + i) * LDK + j0, kf[i] * run);
      store4(sQg + (rg * RPG + i) * LDK + j0, q4 * run);
    }
    f32x4 sfx = one;
#pragma unroll
    for (int i = RPG - 1; i >= 0; --i) {
      store4(sKD + (rg * RPG + i) * LDK + j0, kf[i] * (cs * sfx));
      store4(sKi + (rg * RPG + i) * LDK + j0, kf[i] * (bs * sfx));
      sfx *= gr[i];
    }
    f32x4 bd[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bd[a] = one;
#pragma unroll
      for (int r2 = a * GPB; r2 < (a + 1) * GPB; ++r2) bd[a] *= tots[r2];
    }
    auto rcp4 = [](f32x4 x) {
      return f32x4{__builtin_amdgcn_rcpf(x[0]), __builtin_amdgcn_rcpf(x[1]),
                   __builtin_amdgcn_rcpf(x[2]), __builtin_amdgcn_rcpf(x[3])};
    };
    if (rg < 7) {
      f32x4 pv = bd[1] * bd[2];
      if (rg < 4) pv = rcp4(rg == 0 ? bd[0] : rg == 1 ? bd[1] : rg == 2 ? bd[2] : bd[3]);
      else if (rg == 4) pv = bd[1];
      else if (rg == 5) pv = bd[2];
      store4(sPair + rg * DK + j0, pv);
    }
    if (rg < 4) {
      const f32x4 ec = rg == 0 ? one : rg == 1 ? bd[0] : rg == 2 ? bd[0] * bd[1] : bd[0] * bd[1] * bd[2];
      store4(sEc + rg * DK + j0, ec);
    }
    (void)n;
  }

  // QSCALE: Qg includes the query scale (the backward's chain tiles use it); without it
  // the consumer applies the scale to each output tile instead (one multiply per output
  // element rather than one per Qg element).
  //
  // Strong decay.  The factors above are referenced to the chunk start, so Ki carries
  // e^{-G_r}: past a per-chunk sum of |g| of about 87 it overflows fp32 and A turns
  // into NaN.  A chunk in which some 8-row group of some channel decays by more than
  // e^{-10} (so the chunk sum may exceed 80) is factored per 16-row block instead:
  // Kg and Qg relative to the start of their block, Ki relative to its end, every
  // stored factor <= 1.  The products then scale the Ki fragment of block pair (a, b)
  // by e^{G_{16a-1} - G_{16b+15}} (the decay of the blocks between; 1 / the block's own
  // decay for a = b), and the published Qg and the Kg operand of W get the block-start
  // decay e^{G_{16a-1}} back.  Values are exact in either form (up to rounding); the
  // strong form holds while no 16-row block decays by more than about e^{-85} in a
  // channel.  tag: a number unique to this chunk among this workgroup's chunks.
  template <int DECAY, bool QSCALE = true>
  __device__ __forceinline__ void factors(int n, int tag) {
    unpack_pairs();
    if (flags & kNormK) normalise_keys();
    if constexpr (DECAY == 1) {
      // one log-decay per (row, head): lane l holds row l's, turns it into the decay
      // factor once (rows past the end: 1) and each thread reads the rows of its group
      // from the lanes that hold them
      float x = gr[0][0];
      if (flags & kGateLogit) x = log_sigmoid_hw(x);
      const int a = __builtin_bit_cast(int, lane < n ? exp_hw(x) : 1.f);
      constexpr int GW = 64 / CG;   // row groups per wave
      static_assert(64 % CG == 0, "row groups within a wave");
      const int r0 = __builtin_amdgcn_readfirstlane(tid >> 6) * GW * RPG;
      const int sub = lane / CG;
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        int y = __builtin_amdgcn_readlane(a, r0 + i);
#pragma unroll
        for (int s = 1; s < GW; ++s) {
          const int ys = __builtin_amdgcn_readlane(a, r0 + s * RPG + i);
          y = sub == s ? ys : y;
        }
        const float f = __builtin_bit_cast(float, y);
        gr[i] = f32x4{f, f, f, f};
      }
    }
    // retention logits to log-decays (no decay: alpha = 1 whatever the flag says)
    if (DECAY == 0 && (flags & kGateLogit)) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) gr[i] = log_sigmoid4(gr[i]);
    }
    // Rows past the end of a partial chunk (they re-read the last row): k, q, v zero and
    // g zero (alpha = 1).  Only a sequence's last chunk takes this branch, so full
    // chunks run without per-element masks.
    if (n < kChunk) {
      const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
      const bf16x4 zb = bf16x4{static_cast<bf16>(0.f), static_cast<bf16>(0.f),
                               static_cast<bf16>(0.f), static_cast<bf16>(0.f)};
#pragma unroll
      for (int i = 0; i < RPG; ++i)
        if (rg * RPG + i >= n) {
          if constexpr (DECAY != 1) gr[i] = z;
          kr[i] = zb;
          qr[i] = zb;
        }
#pragma unroll
      for (int i = 0; i < RPGV; ++i)
        if (rgv * RPGV + i >= n) vr[i] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    // alpha = e^g in place (one per row and head: already done); per-thread product
    // of its rows.  With one decay per (row, head) every channel of a row carries the
    // same factor, so its running products are kept as scalars (the same products in
    // the same order as the per-channel form, so the tiles are bit for bit those of a
    // per-channel g broadcast over the channels); with no decay every factor is 1 and
    // the tiles are the inputs themselves.
    [[maybe_unused]] f32x4 tot = f32x4{1.f, 1.f, 1.f, 1.f};
    [[maybe_unused]] float tot1 = 1.f;
    if constexpr (DECAY == 0) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const f32x4 gg = gr[i];
        gr[i] = f32x4{exp_hw(gg[0]), exp_hw(gg[1]), exp_hw(gg[2]), exp_hw(gg[3])};
        tot *= gr[i];
      }
      store4(sScr + rg * DK + j0, tot);
    } else if constexpr (DECAY == 1) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) tot1 *= gr[i][0];
      if (j0 == 0) sScr[rg * DK] = tot1;
    }
    if constexpr (DECAY != 2) {
      constexpr float kStrongTot = 4.5399930e-05f;   // e^{-10}
      const float tmin = DECAY == 1 ? tot1 : min(min(tot[0], tot[1]), min(tot[2], tot[3]));
      if (tmin < kStrongTot) *sStrong = tag;
    }
    if (tid < kChunk)
      sBeta[tid] = tid < n ? ((flags & kBetaLogit) ? sigmoid_hw(br) : br) : 0.f;
    // V rows meanwhile
#pragma unroll
    for (int i = 0; i < RPGV; ++i)
      *reinterpret_cast<u32x4*>(sV + (rgv * RPGV + i) * LDV + jv0) = __builtin_bit_cast(u32x4, vr[i]);
    lds_barrier();
    if constexpr (DECAY == 2) {
      // Kg = Ki = KD = k and Qg = q (times the scale with QSCALE): the input rows as
      // loaded; e^{G_n} = 1
      strong = false;
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const int r = (rg * RPG + i) * LDK + j0;
        *reinterpret_cast<bf16x4*>(sKg + r) = kr[i];
        *reinterpret_cast<bf16x4*>(sKD + r) = kr[i];
        *reinterpret_cast<bf16x4*>(sKi + r) = kr[i];
        if constexpr (QSCALE)
          store4(sQg + r, widen(qr[i]) * scale);
        else
          *reinterpret_cast<bf16x4*>(sQg + r) = qr[i];
      }
      if (rg == 0) store4(sEgn + j0, f32x4{1.f, 1.f, 1.f, 1.f});
      return;
    } else if constexpr (DECAY == 1) {
      strong = __builtin_amdgcn_readfirstlane(*sStrong == tag ? 1 : 0) != 0;
      float tt[RG];
#pragma unroll
      for (int r2 = 0; r2 < RG; ++r2) tt[r2] = sScr[r2 * DK];
      float cp = 1.f, cs = 1.f;
#pragma unroll
      for (int r2 = 0; r2 < RG; ++r2) {
        if (r2 < rg) cp *= tt[r2];
        if (r2 > rg) cs *= tt[r2];
      }
      const float egn = cp * tot1 * cs;   // e^{G_n}
      if (strong) {
        f32x4 tots[RG];
#pragma unroll
        for (int r2 = 0; r2 < RG; ++r2) tots[r2] = f32x4{tt[r2], tt[r2], tt[r2], tt[r2]};
        strong_factors<QSCALE>(tots, f32x4{cs, cs, cs, cs}, n);
        if (rg == 0) store4(sEgn + j0, f32x4{egn, egn, egn, egn});
        return;
      }
      f32x4 kf[RPG];
      float run = cp;
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        run *= gr[i][0];
        kf[i] = widen(kr[i]);
        f32x4 q4 = widen(qr[i]);
        if constexpr (QSCALE) q4 *= scale;
        store4(sKg + (rg * RPG + i) * LDK + j0, kf[i] * run);
        store4(sQg + (rg * RPG + i) * LDK + j0, q4 * run);
      }
      const float rn = __builtin_amdgcn_rcpf(egn);
      float sfx = cs;
#pragma unroll
      for (int i = RPG - 1; i >= 0; --i) {
        const f32x4 kd = kf[i] * sfx;
        store4(sKD + (rg * RPG + i) * LDK + j0, kd);
        store4(sKi + (rg * RPG + i) * LDK + j0, kd * rn);
        sfx *= gr[i][0];
      }
      if (rg == 0) store4(sEgn + j0, f32x4{egn, egn, egn, egn});
      return;
    }
    strong = __builtin_amdgcn_readfirstlane(*sStrong == tag ? 1 : 0) != 0;
    f32x4 tots[RG];
#pragma unroll
    for (int r2 = 0; r2 < RG; ++r2) tots[r2] = *reinterpret_cast<const f32x4*>(sScr + r2 * DK + j0);
    f32x4 cp = f32x4{1.f, 1.f, 1.f, 1.f}, cs = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int r2 = 0; r2 < RG; ++r2) {
      if (r2 < rg) cp *= tots[r2];
      if (r2 > rg) cs *= tots[r2];
    }
    const f32x4 egn = cp * tot * cs;   // e^{G_n}
    if (strong) {
      strong_factors<QSCALE>(tots, cs, n);
      if (rg == 0) store4(sEgn + j0, egn);
      return;
    }
    // forward: e^{G_r} = cp * alpha_first .. alpha_r  ->  Kg, Qg
    f32x4 kf[RPG];
    {
      f32x4 run = cp;
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        run *= gr[i];
        kf[i] = widen(kr[i]);
        f32x4 q4 = widen(qr[i]);
        if constexpr (QSCALE) q4 *= scale;
        store4(sKg + (rg * RPG + i) * LDK + j0, kf[i] * run);
        store4(sQg + (rg * RPG + i) * LDK + j0, q4 * run);
      }
    }
    // backward: e^{G_n - G_r} = alpha_{r+1} .. alpha_n (a suffix product)  ->  KD;
    // Ki = KD / e^{G_n}
    {
      const f32x4 rn = f32x4{__builtin_amdgcn_rcpf(egn[0]), __builtin_amdgcn_rcpf(egn[1]),
                             __builtin_amdgcn_rcpf(egn[2]), __builtin_amdgcn_rcpf(egn[3])};
      f32x4 sfx = cs;
#pragma unroll
      for (int i = RPG - 1; i >= 0; --i) {
        const f32x4 kd = kf[i] * sfx;
        store4(sKD + (rg * RPG + i) * LDK + j0, kd);
        store4(sKi + (rg * RPG + i) * LDK + j0, kd * rn);
        sfx *= gr[i];
      }
    }
    if (rg == 0) store4(sEgn + j0, egn);
  }

  // M^T tiles (a, B0) for a <= B0 and (a, B1) for a <= B1 (Ki rows a, Qg rows b): every
  // fragment of the four K steps is read before the products.
  template <int B0, int B1>
  __device__ __forceinline__ void mt_blocks(f32x4 (&acc)[5]) const {
    bf16x8 q0[KS], q1[KS], ki[KS][B1 + 1];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      q0[t] = frag_rows<M>(sQg, LDK, 16 * B0, 32 * t, lane);
      q1[t] = frag_rows<M>(sQg, LDK, 16 * B1, 32 * t, lane);
#pragma unroll
      for (int a = 0; a <= B1; ++a) ki[t][a] = frag_rows<M>(sKi, LDK, 16 * a, 32 * t, lane);
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KS; ++t) {
#pragma unroll
      for (int a = 0; a <= B0; ++a) acc[a] = mma_bf16(ki[t][a], q0[t], acc[a]);
#pragma unroll
      for (int a = 0; a <= B1; ++a) acc[B0 + 1 + a] = mma_bf16(ki[t][a], q1[t], acc[B0 + 1 + a]);
    }
  }

  // Block-pair factor rows of sPair (see strong_factors).
  static constexpr int kInv0 = 0, kBd1 = 4, kBd2 = 5, kBd12 = 6;
  // Strong-decay forms of lower_blocks (A, waves 0, 1) and mt_blocks (M^T, waves 2, 3):
  // the Ki fragment of block b, paired with block a, times the factors of (a, b).
  // RA = 0: pairs (0,0) (3,0) (3,1) (3,2) (3,3); RA = 1: (1,0) (1,1) (2,0) (2,1) (2,2).
  template <int RA>
  __device__ __forceinline__ void scaled_ki(const bf16x8 (&ki)[4], int kk, bf16x8 (&out)[5]) const {
    const float* pf = sPair + kk + 8 * (lane >> 4);
    if constexpr (RA == 0) {
      out[0] = scale_rows8(ki[0], pf + (kInv0 + 0) * DK);
      out[1] = scale_rows8(ki[0], pf + kBd12 * DK);
      out[2] = scale_rows8(ki[1], pf + kBd2 * DK);
      out[3] = ki[2];
      out[4] = scale_rows8(ki[3], pf + (kInv0 + 3) * DK);
    } else {
      out[0] = ki[0];
      out[1] = scale_rows8(ki[1], pf + (kInv0 + 1) * DK);
      out[2] = scale_rows8(ki[0], pf + kBd1 * DK);
      out[3] = ki[1];
      out[4] = scale_rows8(ki[2], pf + (kInv0 + 2) * DK);
    }
  }
  // A blocks of row blocks (RA, RB) = (0, 3) or (1, 2), as lower_blocks.
  template <int RA, int RB>
  __device__ __forceinline__ void lower_blocks_strong(f32x4 (&acc)[5]) const {
#pragma unroll
    for (int i = 0; i < 5; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK; kk += 32) {
      const bf16x8 a0 = frag_rows<M>(sKg, LDK, 16 * RA, kk, lane);
      const bf16x8 a1 = frag_rows<M>(sKg, LDK, 16 * RB, kk, lane);
      bf16x8 ki[4], b[5];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) ki[cb] = frag_rows<M>(sKi, LDK, 16 * cb, kk, lane);
      scaled_ki<RA>(ki, kk, b);
#pragma unroll
      for (int s = 0; s < 5; ++s) acc[s] = mma_bf16(s <= RA ? a0 : a1, b[s], acc[s]);
    }
  }
  // M^T tiles (a, B0), (a, B1) as mt_blocks; (B0, B1) = (0, 3) or (1, 2) pairs with
  // the same blocks as lower_blocks_strong<B0, B1>.
  template <int B0, int B1>
  __device__ __forceinline__ void mt_blocks_strong(f32x4 (&acc)[5]) const {
#pragma unroll
    for (int i = 0; i < 5; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK; kk += 32) {
      const bf16x8 q0 = frag_rows<M>(sQg, LDK, 16 * B0, kk, lane);
      const bf16x8 q1 = frag_rows<M>(sQg, LDK, 16 * B1, kk, lane);
      bf16x8 ki[4], b[5];
#pragma unroll
      for (int a = 0; a < 4; ++a) ki[a] = frag_rows<M>(sKi, LDK, 16 * a, kk, lane);
      scaled_ki<B0>(ki, kk, b);
      // tile (a, B) = Ki_a Qg_B^T: acc[0..B0] = (a, B0), acc[B0 + 1 + a] = (a, B1)
#pragma unroll
      for (int s = 0; s < 5; ++s) acc[s] = mma_bf16(b[s], s <= B0 ? q0 : q1, acc[s]);
    }
  }

  // Waves 0, 1: A = strict-lower(diag(beta) Kg Ki^T) into LDS (fp32).
  // Waves 2, 3: M^T = Ki Qg^T (tiles (a, b), a <= b, masked to a row <= column) and
  // its M fragments straight to the ring slot.  No closing barrier.
  // TILES: waves 2, 3 also write M itself, row-major bf16 [64][64], to mt (global; the
  // blocks on and below the diagonal, masked as published).
  template <bool TILES = false>
  __device__ __forceinline__ void products(__amdgpu_buffer_rsrc_t rr, uint32_t slot,
                                           bf16* mt = nullptr) {
    const int lq = lane >> 4, lr = lane & 15;
    f32x4 acc[5];
    if (wave < 2) {
      const f32x4 bta = *reinterpret_cast<const f32x4*>(sBeta + 16 * (wave ? 1 : 0) + 4 * lq);
      const f32x4 btb = *reinterpret_cast<const f32x4*>(sBeta + 16 * (wave ? 2 : 3) + 4 * lq);
      if (wave == 0) {
        if (strong)
          lower_blocks_strong<0, 3>(acc);
        else
          lower_blocks<M, DK, LDK, 0, 3>(acc, sKg, sKi, lane);
        store_lower_blocks<true, bf16, LDF, LDC, 0, 3>(acc, bta, btb, sA, nullptr, lane);
      } else {
        if (strong)
          lower_blocks_strong<1, 2>(acc);
        else
          lower_blocks<M, DK, LDK, 1, 2>(acc, sKg, sKi, lane);
        store_lower_blocks<true, bf16, LDF, LDC, 1, 2>(acc, bta, btb, sA, nullptr, lane);
      }
      return;
    }
    // token blocks b of this wave: (0, 3) or (1, 2); tiles (a, b) for a <= b:
    // acc[0..b0] = tiles (a, b0), acc[b0+1 .. b0+1+b1] = tiles (a, b1)
    if (wave == 2) {
      if (strong)
        mt_blocks_strong<0, 3>(acc);
      else
        mt_blocks<0, 3>(acc);
    } else {
      if (strong)
        mt_blocks_strong<1, 2>(acc);
      else
        mt_blocks<1, 2>(acc);
    }
    // causal mask on the diagonal tiles: row (token') 4*lq + i <= column (token) lr
    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
    auto diag = [&](f32x4 t) {
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = 4 * lq + i <= lr ? t[i] : 0.f;
      return r;
    };
    const uint32_t base = slot + SL::oM + 16 * lane;
    if (wave == 2) {
      // b = 0: fragment (0, 0) = tiles (0, 0)diag, (1, 0) = 0
      st16(rr, base + 0 * SL::kFrag, pack_frag(diag(acc[0]), z));
      // b = 3: fragments (3, 0) = tiles (0, 3), (1, 3); (3, 1) = (2, 3), (3, 3)diag
      st16(rr, base + 3 * SL::kFrag, pack_frag(acc[1], acc[2]));
      st16(rr, base + 5 * SL::kFrag, pack_frag(acc[3], diag(acc[4])));
    } else {
      // b = 1: fragment (1, 0) = tiles (0, 1), (1, 1)diag
      st16(rr, base + 1 * SL::kFrag, pack_frag(acc[0], diag(acc[1])));
      // b = 2: fragments (2, 0) = tiles (0, 2), (1, 2); (2, 1) = (2, 2)diag, 0
      st16(rr, base + 2 * SL::kFrag, pack_frag(acc[2], acc[3]));
      st16(rr, base + 4 * SL::kFrag, pack_frag(diag(acc[4]), z));
    }
    if constexpr (TILES) {
      // tile (a, b) holds M[16 b + lr][16 a + 4 lq + i]
      auto put = [&](int ta, int tb, f32x4 t) {
        __builtin_nontemporal_store(
            bf16x4{static_cast<bf16>(t[0]), static_cast<bf16>(t[1]), static_cast<bf16>(t[2]),
                   static_cast<bf16>(t[3])},
            reinterpret_cast<bf16x4*>(mt + (16 * tb + lr) * kChunk + 16 * ta + 4 * lq));
      };
      if (wave == 2) {
        put(0, 0, diag(acc[0]));
        put(0, 3, acc[1]);
        put(1, 3, acc[2]);
        put(2, 3, acc[3]);
        put(3, 3, diag(acc[4]));
      } else {
        put(0, 1, acc[0]);
        put(1, 1, diag(acc[1]));
        put(0, 2, acc[2]);
        put(1, 2, acc[3]);
        put(2, 2, diag(acc[4]));
      }
    }
  }

  // All waves: wave b inverts diagonal block b of I + A (unit lower triangular) by
  // right-looking substitution.  Lane 4c + q owns column c and rows q, q + 4, q + 8,
  // q + 12 of the block; at step j the finished entry x_j of column c is broadcast
  // within the lane's quad (DPP) and every row below subtracts A[r][j] x_j (A holds
  // zeros on and above its diagonal, so rows above j are left as they are).  The
  // dependent chain is 16 steps of one broadcast and one FMA.  X_bb goes to sX (fp32)
  // and, times diag(beta), to sTm (bf16).  No closing barrier.
  __device__ __forceinline__ void inverse_blocks() {
    const int b = wave, c = lane >> 2, q = lane & 3;
    const float* Ab = sA + (16 * b + q) * LDF + 16 * b;
    // a[m][j4] = A[4 m + q][4 j4 .. 4 j4 + 3]: columns past 4 m + 3 are zero for every q
    f32x4 a[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j4 = 0; j4 <= m; ++j4)
        a[m][j4] = *reinterpret_cast<const f32x4*>(Ab + 4 * m * LDF + 4 * j4);
    float x[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) x[m] = 4 * m + q == c ? 1.f : 0.f;
    static_for<15>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const float xj = __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[j >> 2]), (j & 3) * 0x55,
                                          0xf, 0xf, false));
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (4 * m + 3 > j) x[m] = __builtin_fmaf(-a[m][j >> 2][j & 3], xj, x[m]);
    });
    const float bc = sBeta[16 * b + c];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * b + 4 * m + q;
      sX[r * LDF + 16 * b + c] = x[m];
      sTm[r * LDC + 16 * b + c] = static_cast<bf16>(x[m] * bc);
    }
  }

  // Waves 0, 1, after a barrier that follows inverse_blocks: X_10 = -X_11 A_10 X_00
  // (wave 0) or X_32 = -X_33 A_32 X_22 (wave 1), to sX and, times diag(beta), sTm.
  // No closing barrier.
  __device__ __forceinline__ void inverse_pairs() {
    const int lr = lane & 15, lq = lane >> 4;
    const int rb = 2 * wave + 1, cb = 2 * wave;
    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
    // Y = A_10 X_00 lands in accumulator layout, the B operand of X_11 Y as it is
    const f32x4 y = mm16p(z, sA + 16 * rb * LDF + 16 * cb, LDF,
                          acc_layout(sX + 16 * cb * LDF + 16 * cb, LDF, lane), lane);
    const f32x4 x = mm16p(z, sX + 16 * rb * LDF + 16 * rb, LDF, y, lane);
    const float bc = sBeta[16 * cb + lr];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * lq + i;
      sX[r * LDF + 16 * cb + lr] = -x[i];
      sTm[r * LDC + 16 * cb + lr] = static_cast<bf16>(-x[i] * bc);
    }
  }

  // All waves, after a barrier that follows inverse_pairs: the 32x32 block below the
  // diagonal, X_lo = -X_B11 (A_lo X_B00); wave w forms block (w/2, w%2).  Ends with
  // a barrier (Tm complete).
  __device__ __forceinline__ void inverse_rest() {
    const int lr = lane & 15, lq = lane >> 4;
    float* sY = sScr;
    const int bi = 2 + (wave >> 1), bj = wave & 1;
    {
      // both waves of a block row read their operands before either product
      const f32x4 b1 = acc_layout(sX + 16 * LDF + 16 * bj, LDF, lane);
      const f32x4 b0 = acc_layout(sX + 16 * bj, LDF, lane);
      f32x4 y = mm16p(f32x4{0.f, 0.f, 0.f, 0.f}, sA + (16 * bi) * LDF + 16, LDF, b1, lane);
      if (bj == 0) y = mm16p(y, sA + (16 * bi) * LDF, LDF, b0, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) sY[wave * 16 * 17 + (4 * lq + i) * 17 + lr] = y[i];
    }
    lds_barrier();
    {
      const f32x4 y2 = acc_layout(sY + bj * 16 * 17, 17, lane);
      const f32x4 y3 = acc_layout(sY + (2 + bj) * 16 * 17, 17, lane);
      f32x4 x = mm16p(f32x4{0.f, 0.f, 0.f, 0.f}, sX + (16 * bi) * LDF + 32, LDF, y2, lane);
      if (bi == 3) x = mm16p(x, sX + (16 * bi) * LDF + 48, LDF, y3, lane);
      const float bc = sBeta[16 * bj + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * lq + i, c = 16 * bj + lr;
        sTm[r * LDC + c] = static_cast<bf16>(-x[i] * bc);
      }
    }
    lds_barrier();
  }

  // Waves W0 .. W0 + NW - 1: Qg and KD^T fragments and e^{G_n} to the slot.  Wave
  // w' = wave - W0 takes Qg fragments w', w' + NW, ... and then KD^T fragments w',
  // w' + NW, ...; the trip counts are compile-time (indices past the end repeat the
  // last fragment, an identical store), so each wave's reads and stores overlap.
  template <int W0, int NW>
  __device__ __forceinline__ void publish_qk(__amdgpu_buffer_rsrc_t rr, uint32_t slot) {
    constexpr int nQ = 4 * KS, nKD = 2 * (DK / 16);
    constexpr int TQ = (nQ + NW - 1) / NW, TK = (nKD + NW - 1) / NW;
    const int w1 = wave - W0;
    bf16x8 fq[TQ], fk[TK];
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      const int f = min(w1 + NW * i, nQ - 1), tb = f / KS, j = f % KS;
      fq[i] = frag_perm(sQg, LDK, 16 * tb, 32 * j, lane);
      // strong decay: Qg from its block start back to the chunk start
      if (strong) fq[i] = scale_perm8(fq[i], sEc + tb * DK + 32 * j + 4 * (lane >> 4));
    }
#pragma unroll
    for (int i = 0; i < TK; ++i) {
      const int f = min(w1 + NW * i, nKD - 1), kb = f >> 1, t = f & 1;
      fk[i] = frag_tr_perm(sKD, LDK, 32 * t, 16 * kb, lane);
    }
#pragma unroll
    for (int i = 0; i < TQ; ++i)
      st16(rr, slot + SL::oQ + min(w1 + NW * i, nQ - 1) * SL::kFrag + 16 * lane, fq[i]);
#pragma unroll
    for (int i = 0; i < TK; ++i)
      st16(rr, slot + SL::oKD + min(w1 + NW * i, nKD - 1) * SL::kFrag + 16 * lane, fk[i]);
    const int e = tid - 64 * W0;
    if (e >= 0 && e < DK) st4(rr, slot + SL::oEgn + 4 * e, sEgn[e]);
  }

  // publish_wu for d_k = d_v = 128: wave w forms the W fragments (tb, j = w) and the U
  // tiles of value-block pair w for the four token blocks tb.  Every LDS operand is read
  // first -- the products of one token block share its X diag(beta) fragments, those of
  // one K step share the Kg^T and V^T fragments -- then the 24 products run back to back
  // and the eight fragments leave as 16-byte stores.
  __device__ __forceinline__ void publish_wu_128(__amdgpu_buffer_rsrc_t rr, uint32_t slot) {
    static_assert(KS == 4 && SL::NVB / 2 == 4, "one W K step and one U pair per wave");
    bf16x8 xb[4][2], kt[2][2], vt[2][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int t = 0; t < (tb < 2 ? 1 : 2); ++t) xb[tb][t] = frag_rows<M>(sTm, LDC, 16 * tb, 32 * t, lane);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        kt[t][hb] = frag_tr(sKg, LDK, 32 * t, 32 * wave + 16 * hb, lane);
        vt[t][hb] = frag_tr(sV, LDV, 32 * t, 16 * (2 * wave + hb), lane);
      }
    if (strong) {
      // Kg from its block start back to the chunk start: lane l's eight rows lie in
      // block 2t + l / 32, its column is key 32 w + 16 hb + l % 16
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          kt[t][hb] = scale_all(kt[t][hb], sEc[(2 * t + (lane >> 5)) * DK + 32 * wave + 16 * hb + (lane & 15)]);
    }
    f32x4 w[4][2], u[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) w[tb][hb] = u[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // W first, its stores while the U products run
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int t = 0; t < (tb < 2 ? 1 : 2); ++t)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) w[tb][hb] = mma_bf16(kt[t][hb], xb[tb][t], w[tb][hb]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int t = 0; t < (tb < 2 ? 1 : 2); ++t)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) u[tb][hb] = mma_bf16(xb[tb][t], vt[t][hb], u[tb][hb]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      st16(rr, slot + SL::oW + (tb * KS + wave) * SL::kFrag + 16 * lane, pack_frag(-w[tb][0], -w[tb][1]));
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      st16(rr, slot + SL::oU + (tb * (SL::NVB / 2) + wave) * SL::kFrag + 16 * lane,
           pack_frag(u[tb][0], u[tb][1]));
  }

  // Strong decay: Qg in LDS from block-start to chunk-start reference (for readers
  // after the products, the backward's chain tiles).  No closing barrier.
  __device__ __forceinline__ void qg_to_chunk_start() {
    if (!strong) return;
    for (int e = tid; e < kChunk * (DK / 4); e += kThreads) {
      const int r = e / (DK / 4), c = 4 * (e % (DK / 4));
      bf16x4* p = reinterpret_cast<bf16x4*>(sQg + r * LDK + c);
      const f32x4 x = widen(*p) * *reinterpret_cast<const f32x4*>(sEc + (r / 16) * DK + c);
      *p = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                  static_cast<bf16>(x[3])};
    }
  }

  // All waves: W^T = -(Kg^T (X diag(beta))^T) as W fragments and U = X diag(beta) V as
  // fp32 tiles, straight to the slot.  Row block tb of X diag(beta) is zero beyond
  // column 16 tb + 15, so tb < 2 needs one K step.
  // TILES: also -W itself, bf16 rows of LDK, to wt (LDS).
  template <bool TILES = false>
  __device__ __forceinline__ void publish_wu(__amdgpu_buffer_rsrc_t rr, uint32_t slot,
                                             bf16* wt = nullptr) {
    if constexpr (DK == 128 && DV == 128 && !TILES) {
      publish_wu_128(rr, slot);
      return;
    }
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int f = wave + 4 * i, tb = f / KS, j = f % KS;
      f32x4 lo = f32x4{0.f, 0.f, 0.f, 0.f}, hi = lo;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t == 1 && tb < 2) break;
        const bf16x8 xb = frag_rows<M>(sTm, LDC, 16 * tb, 32 * t, lane);
        bf16x8 k0 = frag_tr(sKg, LDK, 32 * t, 32 * j, lane);
        bf16x8 k1 = frag_tr(sKg, LDK, 32 * t, 32 * j + 16, lane);
        if (strong) {   // as in publish_wu_128
          const float* ec = sEc + (2 * t + (lane >> 5)) * DK + 32 * j + (lane & 15);
          k0 = scale_all(k0, ec[0]);
          k1 = scale_all(k1, ec[16]);
        }
        lo = mma_bf16(k0, xb, lo);
        hi = mma_bf16(k1, xb, hi);
      }
      st16(rr, slot + SL::oW + f * SL::kFrag + 16 * lane, pack_frag(-lo, -hi));
      if constexpr (TILES) {
        // lo holds W[16 tb + l % 16][32 j + 4 (l / 16) + e], hi the keys 16 further
        const int lq = lane >> 4, lr = lane & 15;
        bf16* wr = wt + (16 * tb + lr) * LDK + 32 * j + 4 * lq;
        *reinterpret_cast<bf16x4*>(wr) =
            bf16x4{static_cast<bf16>(-lo[0]), static_cast<bf16>(-lo[1]), static_cast<bf16>(-lo[2]),
                   static_cast<bf16>(-lo[3])};
        *reinterpret_cast<bf16x4*>(wr + 16) =
            bf16x4{static_cast<bf16>(-hi[0]), static_cast<bf16>(-hi[1]), static_cast<bf16>(-hi[2]),
                   static_cast<bf16>(-hi[3])};
      }
    }
    // U: wave w forms value-block pairs w, w + 4, ... (blocks 2p, 2p + 1)
    for (int pv = wave; pv < SL::NVB / 2; pv += 4) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (t == 1 && tb < 2) break;
          const bf16x8 xb = frag_rows<M>(sTm, LDC, 16 * tb, 32 * t, lane);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            acc[hb] = mma_bf16(xb, frag_tr(sV, LDV, 32 * t, 16 * (2 * pv + hb), lane), acc[hb]);
        }
        st16(rr, slot + SL::oU + (tb * (SL::NVB / 2) + pv) * SL::kFrag + 16 * lane,
             pack_frag(acc[0], acc[1]));
      }
    }
  }
};

}  // namespace kda
