// Chunk-local work of the KDA prefill on gfx950, shared by the fused and the
// producer/consumer prefill kernels.
//
// For one chunk of n <= 64 rows of one (sequence, head), with alpha_r = e^{g_r}
// per key channel (the decay of "Kimi Delta Attention: The Linear Attention Behind
// Kimi K2 and Qwen3", "How Kimi Delta Attention works step by step"):
//
//   e^{G_r} = alpha_1 ... alpha_r              (inclusive prefix product)
//   Kg_r = k_r e^{G_r}    Ki_r = k_r e^{-G_r}    Qg_r = scale q_r e^{G_r}
//   A    = strictly-lower(diag(beta) Kg Ki^T)  M = lower-incl(Qg Ki^T)
//   X    = (I + A)^{-1}
//
// These depend on the chunk's inputs only, not on the state.  The state step that
// consumes them is
//   E = X diag(beta) (V - Kg S^T);   O = Qg S^T + M E;   S' = (S + E^T Ki) Diag(e^{G_n}),
// which is the token recurrence unrolled over the chunk (exact up to rounding).
//
// ChunkProducer computes Kg, Qg, Ki (and Ki^T), M and X (as the MFMA operand Tm) into
// the workgroup's LDS with 256 threads (4 waves):
//   factors():  one hardware exp per element gives alpha; e^{G_r} and
//               e^{G_n - G_r} are prefix / suffix products, so e^{-G_r} costs one
//               reciprocal per channel.  The next chunk's g, k, q, beta are then
//               loaded into the registers just consumed (branch-free: rows past the
//               end re-read the last valid row and are masked at use).
//   products(): A and M, 20 16x16 output blocks on MFMA, five independent chains
//               per wave.
//   inverse():  X in fp32, blocked 4 x 16: one wave inverts the four diagonal blocks
//               by left-looking substitution (lane = block column) and forms the two
//               sub-diagonal blocks; the 32x32 block below them follows in two fp32
//               MFMA steps (6 dependent 16x16 products in all).
// bf16 inputs use v_mfma_f32_16x16x32_bf16 (fp32 accumulation) with bf16 LDS
// operands; fp32 inputs use v_mfma_f32_16x16x4_f32 and fp32 operands throughout.
//
// Operand convention: an MFMA A operand is an M x K row-major LDS array, a B operand
// is stored N x K row-major (K contiguous), so both are read with the same fragment
// load.  A 16x16 accumulator holds D[4*(l/16)+i][l%16] in lane l.
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int kChunk = 64;
constexpr int kThreads = 256;

// MFMA flavour per input dtype.
template <typename Tin> struct Mfma;
template <> struct Mfma<bf16> {
  using TC = bf16;                  // operand type in LDS
  using frag = bf16x8;
  using raw4 = bf16x4;              // four input elements as loaded
  static constexpr int KSTEP = 32;  // K per instruction
  static constexpr int KPL = 8;     // K elements per lane
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  using TC = float;
  using frag = float;
  using raw4 = f32x4;
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x4 widen(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 widen(bf16x4 x) {
  return f32x4{static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
               static_cast<float>(x[3])};
}

// Store four consecutive operand elements (fp32 rows are padded by one float, so
// they are written element by element; bf16 rows stay 8-byte aligned).
__device__ __forceinline__ void store4(float* p, f32x4 x) {
  p[0] = x[0];
  p[1] = x[1];
  p[2] = x[2];
  p[3] = x[3];
}
__device__ __forceinline__ void store4(bf16* p, f32x4 x) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]),
                                         static_cast<bf16>(x[2]), static_cast<bf16>(x[3])};
}

// Fragment of a row-major M x K (or N x K) LDS array: lane l reads row row0 + l%16,
// K elements k0 + KPL*(l/16) .. +KPL.
template <typename M>
__device__ __forceinline__ typename M::frag frag_rows(const typename M::TC* base, int ld, int row0,
                                                      int k0, int lane) {
  return *reinterpret_cast<const typename M::frag*>(base + (row0 + (lane & 15)) * ld + k0 +
                                                    M::KPL * (lane >> 4));
}

// Fragment of an operand stored K x N (N contiguous): lane l needs column col0 + l%16,
// K element k0 + l/16.  Only for single-element lanes (fp32).
template <typename M>
__device__ __forceinline__ typename M::frag frag_cols(const typename M::TC* base, int ld, int k0,
                                                      int col0, int lane) {
  static_assert(M::KPL == 1, "strided fragment only for single-element lanes");
  return base[(k0 + (lane >> 4)) * ld + col0 + (lane & 15)];
}

// acc += A16 * B16 for 16x16 fp32 blocks (A row-major with stride lda, B row-major
// K x N with stride ldb), on the fp32 MFMA.
__device__ __forceinline__ f32x4 mm16(f32x4 acc, const float* A, int lda, const float* B, int ldb,
                                      int lane) {
#pragma unroll
  for (int kk = 0; kk < 16; kk += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(lane & 15) * lda + kk + (lane >> 4)],
                                               B[(kk + (lane >> 4)) * ldb + (lane & 15)], acc, 0,
                                               0, 0);
  return acc;
}

// Make this wave's LDS writes visible to its own later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for LDS traffic only.  The workgroup's waves exchange data
// through LDS alone, so the barrier waits for this wave's LDS operations
// (lgkmcnt(0)) and leaves global loads in flight: a full __syncthreads() fence
// would also drain prefetched loads.  The signal fences keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The 10 lower-triangular 16x16 blocks of a 64x64 product, in two row-block pairs
// (RA, RB) = (0, 3) or (1, 2): five blocks per wave, as five independent MFMA chains.
template <typename M, int DK, int LDK, int RA, int RB>
__device__ __forceinline__ void lower_blocks(f32x4 (&acc)[5], const typename M::TC* lhs,
                                             const typename M::TC* rhs, int lane) {
#pragma unroll
  for (int i = 0; i < 5; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < DK; kk += M::KSTEP) {
    const auto a0 = frag_rows<M>(lhs, LDK, 16 * RA, kk, lane);
    const auto a1 = frag_rows<M>(lhs, LDK, 16 * RB, kk, lane);
    typename M::frag bk[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) bk[cb] = frag_rows<M>(rhs, LDK, 16 * cb, kk, lane);
#pragma unroll
    for (int cb = 0; cb <= RA; ++cb) acc[cb] = M::mma(a0, bk[cb], acc[cb]);
#pragma unroll
    for (int cb = 0; cb <= RB; ++cb) acc[RA + 1 + cb] = M::mma(a1, bk[cb], acc[RA + 1 + cb]);
  }
}

// Epilogue of lower_blocks: A (fp32, strictly lower, row r scaled by beta_r) when
// IS_A, else M (operand type, lower including the diagonal).
template <bool IS_A, typename TC, int LDF, int LDC, int RA, int RB>
__device__ __forceinline__ void store_lower_blocks(const f32x4 (&acc)[5], f32x4 bta, f32x4 btb,
                                                   float* sA, TC* sM, int lane) {
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const int rb = s <= RA ? RA : RB;
    const int cb = s <= RA ? s : s - RA - 1;
    const f32x4 bt = s <= RA ? bta : btb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * lq + i, c = 16 * cb + lr;
      if constexpr (IS_A)
        sA[r * LDF + c] = c < r ? acc[s][i] * bt[i] : 0.f;
      else
        sM[r * LDC + c] = from_f32<TC>(c <= r ? acc[s][i] : 0.f);
    }
  }
}

// Byte layout of the chunk-local tiles and scratch in LDS.  KIT = false drops the
// Ki^T copy (kernels that read transposed operands with ds_read_b64_tr_b16).
template <typename Tin, int DK, bool KIT = true>
struct ChunkLayout {
  using TC = typename Mfma<Tin>::TC;
  static constexpr bool kBf16 = sizeof(TC) == 2;
  static constexpr int PADC = kBf16 ? 8 : 1;        // 16 B row pad for bf16, 1 float for fp32
  static constexpr int LDK = DK + PADC;             // [64][DK] tiles (and [BV][DK] snapshots)
  static constexpr int LDC = kChunk + PADC;         // [*][64] operand tiles
  static constexpr int LDF = kChunk + 4;            // fp32 [64][64] (A, inverse), 16 B rows
  static constexpr int LDX = kBf16 ? LDF : LDC;     // fp32 path: the inverse is the operand
  static constexpr bool kKiT = kBf16 && KIT;        // bf16 keeps Ki^T (16 B fragments)
  static constexpr int CG = DK / 4, RG = kThreads / CG, RPG = kChunk / RG;

  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t tileK = size_t(kChunk) * LDK * sizeof(TC);
  static constexpr size_t tileC = size_t(kChunk) * LDC * sizeof(TC);
  static constexpr size_t tileF = size_t(kChunk) * LDF * 4;
  static constexpr size_t oKg = 0;
  static constexpr size_t oQg = al(oKg + tileK);
  static constexpr size_t oKi = al(oQg + tileK);
  static constexpr size_t oKiT = al(oKi + tileK);
  static constexpr size_t oTm = al(oKiT + (kKiT ? size_t(DK) * LDC * sizeof(TC) : 0));
  static constexpr size_t oM = al(oTm + tileC);
  static constexpr size_t oA = al(oM + tileC);
  static constexpr size_t oX = al(oA + tileF);
  static constexpr size_t scrTot = size_t(RG) * DK * 4;
  static constexpr size_t scrY = size_t(4) * 16 * 17 * 4;
  static constexpr size_t oScr = al(oX + (kBf16 ? tileF : 0));
  static constexpr size_t oBeta = al(oScr + (scrTot > scrY ? scrTot : scrY));
  static constexpr size_t oEgn = al(oBeta + kChunk * 4);
  static constexpr size_t kBytes = al(oEgn + DK * 4);
};

// Computes one chunk's tiles into LDS.  Holds the next chunk's inputs in registers.
template <typename Tin, int DK, bool KIT = true>
struct ChunkProducer {
  using M = Mfma<Tin>;
  using TC = typename M::TC;
  using raw4 = typename M::raw4;
  using L = ChunkLayout<Tin, DK, KIT>;
  // The optional fp32 e^{G} tile is key-major, [DK][LDEG]: a key's 64 rows are
  // contiguous, in 16 groups of four rows, and group gr of key j sits at position
  // (gr ^ j ^ (j >> 2)) mod 16.  Four consecutive rows of one key are one 16-byte read.
  // j ^ (j >> 2) takes 16 distinct values over 16 consecutive keys (the readers: keys
  // 16b .. 16b + 15) and over keys 4L + c, L = 0 .. 15 (the writers' keys), so neither
  // side's 16 lanes meet in a bank group.
  static constexpr int LDEG = kChunk;
  static_assert(kChunk == 64, "16 row groups per key");
  __device__ __forceinline__ static int eg_at(int key, int row4) {   // row4: multiple of 4
    return key * LDEG + ((((row4 >> 2) ^ key ^ (key >> 2)) & 15) << 2);
  }
  static constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF, LDX = L::LDX;
  static constexpr int CG = L::CG, RG = L::RG, RPG = L::RPG;

  TC *sKg, *sQg, *sKi, *sKiT, *sTm, *sM;
  float *sA, *sX, *sScr, *sBeta, *sEgn;
  float* sEG = nullptr;     // fp32 e^{G_r} tile [DK][LDEG] (factors<DECAY, true> only)
  const float* g;
  const Tin* k;
  const Tin* q;
  const float* beta;
  int32_t H, h;
  uint32_t rowK;            // elements between token rows of q, k, g
  int tid, lane, wave, rg, j0;
  float scale;
  // the chunk's inputs, loaded ahead
  f32x4 gr[RPG];
  raw4 kr[RPG], qr[RPG];
  float br;
  int32_t flags;   // prologue flags (kNormK, kBetaLogit, kGateLogit)

  __device__ __forceinline__ void init(unsigned char* smem, const Tin* q_, const Tin* k_,
                                       const float* g_, const float* beta_, int32_t H_, int32_t h_,
                                       float scale_, int tid_, int wave_, int32_t flags_) {
    flags = flags_;
    sKg = reinterpret_cast<TC*>(smem + L::oKg);
    sQg = reinterpret_cast<TC*>(smem + L::oQg);
    sKi = reinterpret_cast<TC*>(smem + L::oKi);
    sKiT = reinterpret_cast<TC*>(smem + L::oKiT);
    sTm = reinterpret_cast<TC*>(smem + L::oTm);
    sM = reinterpret_cast<TC*>(smem + L::oM);
    sA = reinterpret_cast<float*>(smem + L::oA);
    sX = L::kBf16 ? reinterpret_cast<float*>(smem + L::oX) : reinterpret_cast<float*>(smem + L::oTm);
    sScr = reinterpret_cast<float*>(smem + L::oScr);
    sBeta = reinterpret_cast<float*>(smem + L::oBeta);
    sEgn = reinterpret_cast<float*>(smem + L::oEgn);
    q = q_;
    k = k_;
    g = g_;
    beta = beta_;
    H = H_;
    h = h_;
    rowK = static_cast<uint32_t>(H_) * DK;
    scale = scale_;
    tid = tid_;
    lane = tid_ & 63;
    wave = wave_;
    rg = tid_ / CG;
    j0 = 4 * (tid_ % CG);
    br = 0.f;
    // upper blocks of Tm and M are never written: zero them once
    for (int i = tid; i < kChunk * LDC; i += kThreads) {
      sTm[i] = from_f32<TC>(0.f);
      sM[i] = from_f32<TC>(0.f);
    }
  }

  // Load rows c0 .. c0+n-1 (n >= 1) of g, k, q, beta into registers.  DECAY: 0 = g per
  // key channel, 1 = one g per (row, head) broadcast to the channels, 2 = no g (zero).
  template <int DECAY>
  __device__ __forceinline__ void load(int64_t c0, int n) {
    const int64_t base = (c0 * H + h) * DK;
    const Tin* kb = k + base;
    const Tin* qb = q + base;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const uint32_t off = static_cast<uint32_t>(min(rg * RPG + i, n - 1)) * rowK + j0;
      if constexpr (DECAY == 0) {
        gr[i] = *reinterpret_cast<const f32x4*>(g + base + off);
      } else if constexpr (DECAY == 1) {
        // lane l loads row l's g; factors() hands the rows to the threads that use them
        if (i == 0) gr[0][0] = g[(c0 + min(lane, n - 1)) * H + h];
      } else {
        gr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      kr[i] = *reinterpret_cast<const raw4*>(kb + off);
      qr[i] = *reinterpret_cast<const raw4*>(qb + off);
    }
    br = beta[(c0 + min(lane, n - 1)) * H + h];
  }

  // Kg, Qg, Ki, Ki^T, beta, e^{G_n} of the loaded chunk (n rows) into LDS; then, if
  // has_next, load rows c1 .. c1+n1-1.  Ends with a barrier.
  // Raw keys to unit keys: row norms over the CG threads of a row group; bf16 keys are
  // rounded to bf16 again (what a caller-side normalisation hands over).
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
      if constexpr (sizeof(TC) == 4)
        kr[i] = k4;
      else
        kr[i] = raw4{static_cast<bf16>(k4[0]), static_cast<bf16>(k4[1]),
                     static_cast<bf16>(k4[2]), static_cast<bf16>(k4[3])};
    }
  }

  // KEEP_EG: also write e^{G_r} (fp32) into sEG, key-major.
  template <int DECAY, bool KEEP_EG = false>
  __device__ __forceinline__ void factors(int n, bool has_next, int64_t c1, int n1) {
    if (flags & kNormK) normalise_keys();
    if constexpr (DECAY == 1) {
      const float x = gr[0][0];
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const float y = __shfl(x, rg * RPG + i);
        gr[i] = f32x4{y, y, y, y};
      }
    }
    // retention logits to log-decays (no decay: alpha = 1 whatever the flag says)
    if (DECAY != 2 && (flags & kGateLogit)) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) gr[i] = log_sigmoid4(gr[i]);
    }
    // alpha = e^g in place (1 for rows past the end); per-thread product of its rows
    f32x4 tot = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const f32x4 gg = gr[i];
      gr[i] = rg * RPG + i < n ? f32x4{exp_hw(gg[0]), exp_hw(gg[1]), exp_hw(gg[2]), exp_hw(gg[3])}
                               : f32x4{1.f, 1.f, 1.f, 1.f};
      tot *= gr[i];
    }
    store4(sScr + rg * DK + j0, tot);
    if (tid < kChunk)
      sBeta[tid] = tid < n ? ((flags & kBetaLogit) ? sigmoid_hw(br) : br) : 0.f;
    lds_barrier();
    // products of the other row groups' totals: before (cp) and after (cs) this one
    f32x4 tots[RG];
#pragma unroll
    for (int r2 = 0; r2 < RG; ++r2) tots[r2] = *reinterpret_cast<const f32x4*>(sScr + r2 * DK + j0);
    f32x4 cp = f32x4{1.f, 1.f, 1.f, 1.f}, cs = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int r2 = 0; r2 < RG; ++r2) {
      if (r2 < rg) cp *= tots[r2];
      if (r2 > rg) cs *= tots[r2];
    }
    const f32x4 egn = cp * tot * cs;                              // e^{G_n}
    // forward pass: e^{G_r} = cp * alpha_{first} ... alpha_r  ->  Kg, Qg
    f32x4 run = cp;
    [[maybe_unused]] f32x4 egr[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const bool ok = rg * RPG + i < n;
      run *= gr[i];
      const f32x4 k4 = ok ? widen(kr[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 q4 = ok ? widen(qr[i]) * scale : f32x4{0.f, 0.f, 0.f, 0.f};
      store4(sKg + (rg * RPG + i) * LDK + j0, k4 * run);
      store4(sQg + (rg * RPG + i) * LDK + j0, q4 * run);
      if constexpr (KEEP_EG) egr[i] = run;
    }
    if constexpr (KEEP_EG) {
      // this thread's rows of each of its four keys: RPG consecutive floats per key
      static_assert(RPG % 4 == 0, "whole 16-byte pieces per key");
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < RPG; i += 4)
          *reinterpret_cast<f32x4*>(sEG + eg_at(j0 + c, rg * RPG + i)) =
              f32x4{egr[i][c], egr[i + 1][c], egr[i + 2][c], egr[i + 3][c]};
    }
    // backward pass: e^{-G_r} = (alpha_{r+1} ... alpha_n) / e^{G_n}  ->  Ki, Ki^T
    run = cs * f32x4{__builtin_amdgcn_rcpf(egn[0]), __builtin_amdgcn_rcpf(egn[1]),
                     __builtin_amdgcn_rcpf(egn[2]), __builtin_amdgcn_rcpf(egn[3])};
    TC kit[4][RPG];
#pragma unroll
    for (int i = RPG - 1; i >= 0; --i) {
      const bool ok = rg * RPG + i < n;
      const f32x4 k4 = ok ? widen(kr[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 ki = k4 * run;
      store4(sKi + (rg * RPG + i) * LDK + j0, ki);
#pragma unroll
      for (int c = 0; c < 4; ++c) kit[c][i] = from_f32<TC>(ki[c]);
      run *= gr[i];
    }
    if constexpr (L::kKiT) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        TC* dst = sKiT + (j0 + c) * LDC + rg * RPG;
        if constexpr (RPG == 8)
          *reinterpret_cast<bf16x8*>(dst) = bf16x8{kit[c][0], kit[c][1], kit[c][2], kit[c][3],
                                                   kit[c][4], kit[c][5], kit[c][6], kit[c][7]};
        else
          *reinterpret_cast<bf16x4*>(dst) = bf16x4{kit[c][0], kit[c][1], kit[c][2], kit[c][3]};
      }
    }
    if (rg == 0) store4(sEgn + j0, egn);
    // the registers are free: load the next chunk's g, k, q, beta
    if (has_next) load<DECAY>(c1, n1);
    lds_barrier();
  }

  // A = strict-lower(diag(beta) Kg Ki^T) (fp32) and M = lower(Qg Ki^T) (operand type).
  // Waves 0, 1: A row blocks (0, 3) and (1, 2); waves 2, 3: the same for M.  Ends with
  // a barrier.
  __device__ __forceinline__ void products() {
    const int lq = lane >> 4;
    f32x4 acc[5];
    const f32x4 bta = *reinterpret_cast<const f32x4*>(sBeta + 16 * ((wave & 1) ? 1 : 0) + 4 * lq);
    const f32x4 btb = *reinterpret_cast<const f32x4*>(sBeta + 16 * ((wave & 1) ? 2 : 3) + 4 * lq);
    if (wave == 0) {
      lower_blocks<M, DK, LDK, 0, 3>(acc, sKg, sKi, lane);
      store_lower_blocks<true, TC, LDF, LDC, 0, 3>(acc, bta, btb, sA, sM, lane);
    } else if (wave == 1) {
      lower_blocks<M, DK, LDK, 1, 2>(acc, sKg, sKi, lane);
      store_lower_blocks<true, TC, LDF, LDC, 1, 2>(acc, bta, btb, sA, sM, lane);
    } else if (wave == 2) {
      lower_blocks<M, DK, LDK, 0, 3>(acc, sQg, sKi, lane);
      store_lower_blocks<false, TC, LDF, LDC, 0, 3>(acc, bta, btb, sA, sM, lane);
    } else {
      lower_blocks<M, DK, LDK, 1, 2>(acc, sQg, sKi, lane);
      store_lower_blocks<false, TC, LDF, LDC, 1, 2>(acc, bta, btb, sA, sM, lane);
    }
    lds_barrier();
  }

  // X = (I + A)^{-1}, written as the operand Tm (bf16, or fp32 in place on the fp32
  // path).  Ends with a barrier.
  __device__ __forceinline__ void inverse() {
    const int lr = lane & 15, lq = lane >> 4;
    float* sY = sScr;   // four 16x17 fp32 scratch blocks
    if (wave == 0) {
      // diagonal blocks, lane = (block b, column c): x = column c of X_bb, row by row
      // (left-looking), each A row read as 16-byte loads
      {
        const int b = lane >> 4, c = lane & 15;
        const float* Ab = sA + (16 * b) * LDF + 16 * b;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
          for (int j4 = 0; j4 < r; j4 += 4) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(Ab + r * LDF + j4);
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (j4 + u < r) acc -= a4[u] * x[j4 + u];
          }
          x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sX[(16 * b + r) * LDX + 16 * b + c] = x[r];
          if constexpr (L::kBf16) sTm[(16 * b + r) * LDC + 16 * b + c] = from_f32<TC>(x[r]);
        }
      }
      wave_lds_sync();
      // X_10 = -X_11 A_10 X_00 and X_32 = -X_33 A_32 X_22
      {
        const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 y0 = mm16(z, sA + 16 * LDF, LDF, sX, LDX, lane);
        const f32x4 y1 = mm16(z, sA + 48 * LDF + 32, LDF, sX + 32 * LDX + 32, LDX, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sY[(4 * lq + i) * 17 + lr] = y0[i];
          sY[16 * 17 + (4 * lq + i) * 17 + lr] = y1[i];
        }
        wave_lds_sync();
        const f32x4 x10 = mm16(z, sX + 16 * LDX + 16, LDX, sY, 17, lane);
        const f32x4 x32 = mm16(z, sX + 48 * LDX + 48, LDX, sY + 16 * 17, 17, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * lq + i;
          sX[(16 + r) * LDX + lr] = -x10[i];
          sX[(48 + r) * LDX + 32 + lr] = -x32[i];
          if constexpr (L::kBf16) {
            sTm[(16 + r) * LDC + lr] = from_f32<TC>(-x10[i]);
            sTm[(48 + r) * LDC + 32 + lr] = from_f32<TC>(-x32[i]);
          }
        }
      }
    }
    lds_barrier();
    // the 32x32 block below the diagonal: X_lo = -X_B11 (A_lo X_B00);
    // wave w computes block (w/2, w%2) of Y = A_lo X_B00, then of X_lo
    const int bi = 2 + (wave >> 1), bj = wave & 1;
    {
      f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb >= bj) y = mm16(y, sA + (16 * bi) * LDF + 16 * kb, LDF,
                               sX + (16 * kb) * LDX + 16 * bj, LDX, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) sY[wave * 16 * 17 + (4 * lq + i) * 17 + lr] = y[i];
    }
    lds_barrier();
    {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 2; kb < 4; ++kb)
        if (kb <= bi) x = mm16(x, sX + (16 * bi) * LDX + 16 * kb, LDX,
                               sY + ((kb - 2) * 2 + bj) * 16 * 17, 17, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * lq + i, c = 16 * bj + lr;
        if constexpr (L::kBf16)
          sTm[r * LDC + c] = from_f32<TC>(-x[i]);
        else
          sX[r * LDX + c] = -x[i];
      }
    }
    lds_barrier();
  }
};

}  // namespace kda
