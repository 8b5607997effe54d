// Chunked KDA prefill on gfx950 (chunk = 64 tokens), fused into one kernel.
//
// Method: the per-token recurrence of "Kimi Delta Attention: The Linear Attention
// Behind Kimi K2 and Qwen3" (elsolitario.org, "How Kimi Delta Attention works step
// by step"), evaluated a chunk at a time; the state at the end of a chunk seeds
// the next ("Kimi Delta Attention Technical Deep Dive", "Systems and
// implementation tradeoffs" -> "Training").  Per chunk of n <= 64 rows, starting
// from the state S (d_v x d_k), with alpha_r = e^{g_r}:
//
//   e^{G_r} = alpha_1 ... alpha_r         (inclusive prefix product per key channel)
//   Kg_r = k_r e^{G_r}      Ki_r = k_r e^{-G_r}      Qg_r = scale q_r e^{G_r}
//   A    = strictly-lower(diag(beta) Kg Ki^T)
//   X    = (I + A)^{-1}                              (unit lower triangular)
//   E    = X diag(beta) (V - Kg S^T)                 (row r = token error e_r)
//   O    = Qg S^T + lower-incl(Qg Ki^T) E
//   S'   = (S + E^T Ki) Diag(e^{G_n})
//
// This is exact (up to rounding) for any chunk size; it follows from unrolling the
// recurrence inside the chunk.  Rows of S (the d_v index) never mix, so each
// (sequence, head) is split into d_v tiles of BV rows that run as independent
// workgroups; the d_v-independent chunk work is recomputed by each tile.
//
// Per chunk, 256 threads (4 waves), one workgroup per (seq, head, v-tile):
//  1. factors: the chunk's g, k, q (loaded one chunk ahead, branch-free) give
//     alpha = e^g with one hardware exp per element; e^{G_r} and e^{G_n - G_r}
//     are prefix / suffix products (so e^{-G_r} = e^{G_n - G_r} / e^{G_n} costs
//     one reciprocal per channel).  Kg, Qg, Ki and Ki^T go to LDS as MFMA operands.
//  2. A and M = lower(Qg Ki^T): 20 16x16 output blocks, 5 independent MFMA chains
//     per wave.
//  3. X = (I + A)^{-1} in fp32, blocked 4 x 16: one wave inverts the four diagonal
//     blocks by right-looking substitution (lane = block column) and forms the two
//     sub-diagonal blocks; the 32x32 off-diagonal super-block follows in two
//     fp32-MFMA steps (6 dependent 16x16 products in all).
//  4. the state step: P = Kg S^T and Qs = Qg S^T; R' = diag(beta)(V - P);
//     E = X R'; O = Qs + M E (stored); S^T <- (S^T + Ki^T E) Diag(e^{G_n}).
//
// The fp32 state tile lives in MFMA accumulators for the whole sequence, held
// transposed (S^T: rows = key channel) so the update lands in the registers that
// hold it; after each chunk a snapshot (bf16 on the bf16 path) goes to LDS as the
// next chunk's operand.  bf16 inputs use v_mfma_f32_16x16x32_bf16 with fp32
// accumulation; fp32 inputs use v_mfma_f32_16x16x4_f32 throughout, so the fp32
// path never rounds to bf16.  The inverse is always built in fp32.
//
// Operand convention: an MFMA A operand is an M x K row-major LDS array, a B
// operand is stored N x K row-major (K contiguous), so both are read with the same
// fragment load.  A 16x16 accumulator holds D[4*(l/16)+i][l%16] in lane l.

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
// would also drain the next chunk's prefetched loads.  The signal fences keep the
// compiler from moving memory operations across it.
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

// Byte layout of the workgroup's LDS.
template <typename Tin, int DK, int BV>
struct Smem {
  using TC = typename Mfma<Tin>::TC;
  static constexpr bool kBf16 = sizeof(TC) == 2;
  static constexpr int PADC = kBf16 ? 8 : 1;        // 16 B row pad for bf16, 1 float for fp32
  static constexpr int LDK = DK + PADC;             // [64][DK] tiles and the [BV][DK] snapshot
  static constexpr int LDC = kChunk + PADC;         // [*][64] operand tiles
  static constexpr int LDF = kChunk + 4;            // fp32 [64][64] (A, inverse), 16 B rows
  static constexpr int LDX = kBf16 ? LDF : LDC;     // fp32 path: the inverse is the operand
  static constexpr bool kKiT = kBf16;               // bf16 keeps Ki^T (16 B fragments)
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
  static constexpr size_t oS = al(oX + (kBf16 ? tileF : 0));
  static constexpr size_t scrTot = size_t(RG) * DK * 4;
  static constexpr size_t scrY = size_t(4) * 16 * 17 * 4;
  static constexpr size_t oScr = al(oS + size_t(BV) * LDK * sizeof(TC));
  static constexpr size_t oBeta = al(oScr + (scrTot > scrY ? scrTot : scrY));
  static constexpr size_t oEgn = al(oBeta + kChunk * 4);
  static constexpr size_t kBytes = al(oEgn + DK * 4);
  // R'^T and E^T ([BV][64]) reuse the A (and fp32 inverse) region, dead by then.
  static constexpr size_t oRT = oA;
  static constexpr size_t oET = al(oRT + size_t(BV) * LDC * sizeof(TC));
  static_assert(oET + size_t(BV) * LDC * sizeof(TC) <= oS, "R^T/E^T overflow their region");
  static_assert(kBytes <= 160 * 1024, "LDS budget exceeded");
};

template <typename Tin, int DK, int BV>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu_seqlens, int64_t T, int32_t H, int32_t DV, int32_t NV,
    int32_t units, int32_t xcd_remap, float scale, const float* initial_state,
    float* final_state, Tin* __restrict__ o) {
  using M = Mfma<Tin>;
  using TC = typename M::TC;
  using raw4 = typename M::raw4;
  using L = Smem<Tin, DK, BV>;
  constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF, LDX = L::LDX;
  constexpr int CG = L::CG, RG = L::RG, RPG = L::RPG;
  constexpr int NVB = BV / 16;                 // 16-wide value blocks in the tile
  constexpr int NST = (DK / 16) * NVB / 4;     // S^T accumulator tiles per wave
  static_assert(NST >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::kBytes];
  TC* sKg = reinterpret_cast<TC*>(smem + L::oKg);
  TC* sQg = reinterpret_cast<TC*>(smem + L::oQg);
  TC* sKi = reinterpret_cast<TC*>(smem + L::oKi);
  TC* sKiT = reinterpret_cast<TC*>(smem + L::oKiT);
  TC* sTm = reinterpret_cast<TC*>(smem + L::oTm);
  TC* sM = reinterpret_cast<TC*>(smem + L::oM);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  float* sX = L::kBf16 ? reinterpret_cast<float*>(smem + L::oX) : reinterpret_cast<float*>(smem + L::oTm);
  TC* sS = reinterpret_cast<TC*>(smem + L::oS);
  float* sScr = reinterpret_cast<float*>(smem + L::oScr);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
  float* sEgn = reinterpret_cast<float*>(smem + L::oEgn);
  TC* sRT = reinterpret_cast<TC*>(smem + L::oRT);
  TC* sET = reinterpret_cast<TC*>(smem + L::oET);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lr = lane & 15;          // accumulator column / fragment row
  const int lq = lane >> 4;          // accumulator row quad

  // ---- work decomposition: workgroup -> (sequence, head, v-tile) ------------------
  int unit, vt;
  {
    const int x = blockIdx.x;
    if (xcd_remap) {
      // consecutive workgroup ids go round-robin to the 8 XCDs; keep the NV tiles of
      // one (seq, head) on one XCD so its q/k/g chunk reads hit that XCD's L2.
      const int xcd = x & 7, y = x >> 3;
      unit = xcd * (units >> 3) + y / NV;
      vt = y % NV;
    } else {
      unit = x / NV;
      vt = x % NV;
    }
  }
  const int n_seq = unit / H, h = unit % H;
  int64_t bos, eos;
  if (cu_seqlens) {
    bos = cu_seqlens[n_seq];
    eos = cu_seqlens[n_seq + 1];
  } else {
    bos = static_cast<int64_t>(n_seq) * T;
    eos = bos + T;
  }
  const int v0 = vt * BV;
  const int cg = tid % CG, rg = tid / CG, j0 = 4 * cg;

  // ---- zero the operand tiles whose upper blocks are never written ---------------
  for (int i = tid; i < kChunk * LDC; i += kThreads) {
    sTm[i] = from_f32<TC>(0.f);
    sM[i] = from_f32<TC>(0.f);
  }

  // ---- initial state -> S^T accumulators ------------------------------------------
  // tile index t = kb * NVB + vb is owned by wave t % 4 (slot t / 4).
  f32x4 sacc[NST];
  const int64_t st_base = (static_cast<int64_t>(n_seq) * H + h) * DV * DK;
#pragma unroll
  for (int s = 0; s < NST; ++s) {
    const int t = wave + 4 * s, kb = t / NVB, vb = t % NVB;
    const int vrow = v0 + 16 * vb + lr, kcol = 16 * kb + 4 * lq;
    if (initial_state)
      sacc[s] = *reinterpret_cast<const f32x4*>(initial_state + st_base + int64_t(vrow) * DK + kcol);
    else
      sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    store4(sS + (16 * vb + lr) * LDK + kcol, sacc[s]);
  }

  // ---- chunk inputs, loaded one chunk ahead into the registers that consumed the
  //      previous chunk (rows past the end re-read the last valid row and are masked
  //      at use, so every load is unconditional).  Addresses are a wave-uniform
  //      chunk base plus 32-bit per-lane offsets.
  const uint32_t rowK = static_cast<uint32_t>(H) * DK;       // elements between token rows
  const uint32_t rowV = static_cast<uint32_t>(H) * DV;
  f32x4 gr[RPG];
  raw4 kr[RPG], qr[RPG];
  uint32_t vr[NVB][4];                // raw value bits (bf16 in the low half, or fp32)
  float br = 0.f;
  auto load_factors = [&](int64_t c0, int n) {
    const int64_t base = (c0 * H + h) * DK;
    const float* gb = g + base;
    const Tin* kb = k + base;
    const Tin* qb = q + base;
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const uint32_t off = static_cast<uint32_t>(min(rg * RPG + i, n - 1)) * rowK + j0;
      gr[i] = *reinterpret_cast<const f32x4*>(gb + off);
      kr[i] = *reinterpret_cast<const raw4*>(kb + off);
      qr[i] = *reinterpret_cast<const raw4*>(qb + off);
    }
    br = beta[(c0 + min(lane, n - 1)) * H + h];
  };
  auto load_values = [&](int64_t c0, int n) {
    const Tin* vb0 = v + (c0 * H + h) * DV + v0;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off =
            static_cast<uint32_t>(min(16 * wave + 4 * lq + i, n - 1)) * rowV + 16 * vb + lr;
        if constexpr (sizeof(Tin) == 2)
          vr[vb][i] = *reinterpret_cast<const unsigned short*>(vb0 + off);
        else
          vr[vb][i] = *reinterpret_cast<const uint32_t*>(vb0 + off);
      }
  };
  auto value_f32 = [&](uint32_t bits) {
    return sizeof(Tin) == 2 ? __uint_as_float(bits << 16) : __uint_as_float(bits);
  };
  if (bos < eos) {
    const int n0 = static_cast<int>(min(eos - bos, static_cast<int64_t>(kChunk)));
    load_factors(bos, n0);
    load_values(bos, n0);
  }

  for (int64_t c0 = bos; c0 < eos; c0 += kChunk) {
    const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
    const int64_t c1 = c0 + kChunk;
    const bool has_next = c1 < eos;
    const int n1 = has_next ? static_cast<int>(min(eos - c1, static_cast<int64_t>(kChunk))) : 0;

    // ---- 1. factor tiles ---------------------------------------------------------
    {
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
      if (tid < kChunk) sBeta[tid] = tid < n ? br : 0.f;
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
      const f32x4 egn = cp * tot * cs;                            // e^{G_n}
      // forward pass: e^{G_r} = cp * alpha_{first} ... alpha_r  ->  Kg, Qg
      f32x4 run = cp;
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const bool ok = rg * RPG + i < n;
        run *= gr[i];
        const f32x4 k4 = ok ? widen(kr[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 q4 = ok ? widen(qr[i]) * scale : f32x4{0.f, 0.f, 0.f, 0.f};
        store4(sKg + (rg * RPG + i) * LDK + j0, k4 * run);
        store4(sQg + (rg * RPG + i) * LDK + j0, q4 * run);
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
      // the registers are free: prefetch the next chunk's g, k, q, beta
      if (has_next) load_factors(c1, n1);
    }
    lds_barrier();

    // ---- 2. A = strict-lower(diag(beta) Kg Ki^T), M = lower(Qg Ki^T) --------------
    //      waves 0, 1: A row blocks (0, 3) and (1, 2); waves 2, 3: the same for M
    {
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
    }
    lds_barrier();

    // ---- 3. X = (I + A)^{-1} ---------------------------------------------------------
    float* sY = sScr;   // four 16x17 fp32 scratch blocks
    if (wave == 0) {
      // 3a: diagonal blocks, lane = (block b, column c): x = column c of X_bb, row by
      //     row (left-looking), each A row read as four 16-byte loads
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
      // 3b: X_10 = -X_11 A_10 X_00 and X_32 = -X_33 A_32 X_22
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
    // 3c: the 32x32 block below the diagonal: X_lo = -X_B11 (A_lo X_B00)
    //     wave w computes Y_w = (A_lo X_B00) block (w/2, w%2)
    {
      const int bi = 2 + (wave >> 1), bj = wave & 1;          // block of A_lo X_B00
      f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
      // sum over k-blocks bj..1 of A[bi][kb] X[kb][bj]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb >= bj) y = mm16(y, sA + (16 * bi) * LDF + 16 * kb, LDF,
                               sX + (16 * kb) * LDX + 16 * bj, LDX, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) sY[wave * 16 * 17 + (4 * lq + i) * 17 + lr] = y[i];
    }
    lds_barrier();
    {
      // wave w: X[2 + w/2][w%2] = -(sum_{kb=2}^{2+w/2} X[2+w/2][kb] Y[kb-2][w%2])
      const int bi = 2 + (wave >> 1), bj = wave & 1;
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

    // ---- 4a. P = Kg S^T, Qs = Qg S^T; R' = diag(beta)(V - P) -> R'^T ----------------
    f32x4 accQ[NVB];
    {
      f32x4 accP[NVB];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) accP[vb] = accQ[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < DK; kk += M::KSTEP) {
        const auto aK = frag_rows<M>(sKg, LDK, 16 * wave, kk, lane);
        const auto aQ = frag_rows<M>(sQg, LDK, 16 * wave, kk, lane);
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const auto bS = frag_rows<M>(sS, LDK, 16 * vb, kk, lane);
          accP[vb] = M::mma(aK, bS, accP[vb]);
          accQ[vb] = M::mma(aQ, bS, accQ[vb]);
        }
      }
      const f32x4 bt = *reinterpret_cast<const f32x4*>(sBeta + 16 * wave + 4 * lq);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 rv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = 16 * wave + 4 * lq + i < n;
          rv[i] = ok ? bt[i] * (value_f32(vr[vb][i]) - accP[vb][i]) : 0.f;
        }
        store4(sRT + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, rv);
      }
      // the value registers are free: prefetch the next chunk's tile
      if (has_next) load_values(c1, n1);
    }
    lds_barrier();

    // ---- 4b. E = X R' -> E^T ---------------------------------------------------------
    {
      const int kend = 16 * (wave + 1);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < kend; kk += M::KSTEP)
          acc = M::mma(frag_rows<M>(sTm, LDC, 16 * wave, kk, lane),
                       frag_rows<M>(sRT, LDC, 16 * vb, kk, lane), acc);
        store4(sET + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, acc);
      }
    }
    lds_barrier();

    // ---- 4c. O = Qs + M E (store); S^T = (S^T + Ki^T E) Diag(e^{G_n}) -----------------
    {
      const int kend = 16 * (wave + 1);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 acc = accQ[vb];
        for (int kk = 0; kk < kend; kk += M::KSTEP)
          acc = M::mma(frag_rows<M>(sM, LDC, 16 * wave, kk, lane),
                       frag_rows<M>(sET, LDC, 16 * vb, kk, lane), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * wave + 4 * lq + i;
          if (r < n) o[((c0 + r) * H + h) * DV + v0 + 16 * vb + lr] = from_f32<Tin>(acc[i]);
        }
      }
#pragma unroll
      for (int s = 0; s < NST; ++s) {
        const int t = wave + 4 * s, kb = t / NVB, vb = t % NVB;
        f32x4 acc = sacc[s];
#pragma unroll
        for (int kk = 0; kk < kChunk; kk += M::KSTEP) {
          typename M::frag a;
          if constexpr (L::kKiT)
            a = frag_rows<M>(sKiT, LDC, 16 * kb, kk, lane);
          else
            a = frag_cols<M>(sKi, LDK, kk, 16 * kb, lane);
          acc = M::mma(a, frag_rows<M>(sET, LDC, 16 * vb, kk, lane), acc);
        }
        const f32x4 e = *reinterpret_cast<const f32x4*>(sEgn + 16 * kb + 4 * lq);
        acc *= e;
        store4(sS + (16 * vb + lr) * LDK + 16 * kb + 4 * lq, acc);
        sacc[s] = acc;
      }
    }
    lds_barrier();
  }

  // ---- final state ------------------------------------------------------------------
  if (final_state) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int t = wave + 4 * s, kb = t / NVB, vb = t % NVB;
      const int vrow = v0 + 16 * vb + lr, kcol = 16 * kb + 4 * lq;
      *reinterpret_cast<f32x4*>(final_state + st_base + int64_t(vrow) * DK + kcol) = sacc[s];
    }
  }
}

template <typename Tin, int DK, int BV>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const int32_t* cu, int64_t T, int32_t H,
                                   int32_t DV, int32_t NV, int32_t units, int32_t xcd_remap,
                                   float scale, const float* s0, float* s1, void* o,
                                   hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<Tin, DK, BV>), dim3(units * NV), dim3(kThreads), 0, stream,
                     static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                     static_cast<const Tin*>(v), g, beta, cu, T, H, DV, NV, units, xcd_remap,
                     scale, s0, s1, static_cast<Tin*>(o));
  return hipGetLastError();
}

// Largest value-tile height each dtype / d_k instantiation supports (LDS budget:
// fp32 operands are twice the size of bf16 ones).
constexpr int max_bv(bool fp32, int dk) { return fp32 ? (dk == 128 ? 16 : 32) : 64; }
int prefill_max_bv(int dtype, int dk) { return max_bv(dtype == 0, dk); }

template <typename Tin, int DK>
static hipError_t launch_prefill_dk(int bv, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const int32_t* cu,
                                    int64_t T, int32_t H, int32_t DV, int32_t NV, int32_t units,
                                    int32_t xcd_remap, float scale, const float* s0, float* s1,
                                    void* o, hipStream_t stream) {
  constexpr int kMax = max_bv(sizeof(Tin) == 4, DK);
  if constexpr (kMax >= 64) {
    if (bv == 64)
      return launch_prefill_t<Tin, DK, 64>(q, k, v, g, beta, cu, T, H, DV, NV, units, xcd_remap,
                                           scale, s0, s1, o, stream);
  }
  if constexpr (kMax >= 32) {
    if (bv == 32)
      return launch_prefill_t<Tin, DK, 32>(q, k, v, g, beta, cu, T, H, DV, NV, units, xcd_remap,
                                           scale, s0, s1, o, stream);
  }
  return launch_prefill_t<Tin, DK, 16>(q, k, v, g, beta, cu, T, H, DV, NV, units, xcd_remap,
                                       scale, s0, s1, o, stream);
}

// Called by the C ABI after validation.  bv in {16, 32, 64} with bv <= prefill_max_bv,
// NV = DV / bv.
hipError_t launch_prefill(int dtype, int dk, int bv, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, const int32_t* cu,
                          int64_t T, int32_t H, int32_t DV, int32_t NV, int32_t units,
                          int32_t xcd_remap, float scale, const float* s0, float* s1, void* o,
                          hipStream_t stream) {
  if (dtype == 1) {
    if (dk == 64)
      return launch_prefill_dk<bf16, 64>(bv, q, k, v, g, beta, cu, T, H, DV, NV, units, xcd_remap,
                                         scale, s0, s1, o, stream);
    return launch_prefill_dk<bf16, 128>(bv, q, k, v, g, beta, cu, T, H, DV, NV, units, xcd_remap,
                                        scale, s0, s1, o, stream);
  }
  if (dk == 64)
    return launch_prefill_dk<float, 64>(bv, q, k, v, g, beta, cu, T, H, DV, NV, units, xcd_remap,
                                        scale, s0, s1, o, stream);
  return launch_prefill_dk<float, 128>(bv, q, k, v, g, beta, cu, T, H, DV, NV, units, xcd_remap,
                                       scale, s0, s1, o, stream);
}

}  // namespace kda
