// Chunked KDA prefill on gfx950 (chunk = 64 tokens), fused into one kernel.
//
// Method: the per-token recurrence of "Kimi Delta Attention: The Linear Attention
// Behind Kimi K2 and Qwen3" (elsolitario.org, "How Kimi Delta Attention works step
// by step"), evaluated a chunk at a time; the state at the end of a chunk seeds
// the next ("Kimi Delta Attention Technical Deep Dive", "Systems and
// implementation tradeoffs" -> "Training").  Per chunk of n <= 64 rows, starting
// from the state S (d_v x d_k):
//
//   G_r  = g_1 + ... + g_r  (inclusive prefix per key channel)
//   Kg_r = k_r e^{G_r}      Ki_r = k_r e^{-G_r}      Qg_r = scale q_r e^{G_r}
//   A    = strictly-lower(diag(beta) Kg Ki^T)
//   Tm   = (I + A)^{-1} diag(beta)                  (forward substitution)
//   E    = Tm (V - Kg S^T)                          (row r = token error e_r)
//   O    = Qg S^T + lower-incl(Qg Ki^T) E
//   S'   = (S + E^T Ki) Diag(e^{G_n})
//
// This is exact (up to rounding) for any chunk size; it follows from unrolling the
// recurrence inside the chunk.  Rows of S (the d_v index) never mix, so each
// (sequence, head) is split into d_v tiles of BV rows that run as independent
// workgroups; the d_v-independent chunk work (prefix, exponentials, A, Tm, M) is
// recomputed by each tile's workgroup.
//
// Layout and roles (256 threads = 4 waves, one workgroup per (seq, head, v-tile)):
//  * The fp32 state tile lives in MFMA accumulators for the whole sequence, held
//    transposed (S^T: rows = key channel, cols = value index) so the update
//    S^T += Ki^T E lands in the registers that hold it; a bf16 (or fp32) snapshot
//    is written to LDS after each chunk as the MFMA operand of the next chunk.
//  * Every contraction is a 16x16 MFMA tile: bf16 inputs use
//    v_mfma_f32_16x16x32_bf16 (fp32 accumulation), fp32 inputs use
//    v_mfma_f32_16x16x4_f32, so the fp32 path never rounds to bf16.
//  * (I + A)^{-1} is blocked 4 x 16: one wave inverts the four 16x16 diagonal
//    blocks (one lane per block column), the off-diagonal blocks follow by fp32
//    MFMA products in three dependency steps.
//
// Operand convention: an MFMA A operand is an M x K row-major LDS array, a B
// operand is stored N x K row-major (K contiguous), so both are read with the same
// 16-byte fragment load.  A 16x16 accumulator holds D[4*(l/16)+i][l%16] in lane l.

#include "kda_device.h"

namespace kda {

constexpr int kChunk = 64;
constexpr int kThreads = 256;

// MFMA flavour per input dtype.
template <typename Tin> struct Mfma;
template <> struct Mfma<bf16> {
  using TC = bf16;                  // operand type in LDS
  using frag = bf16x8;
  static constexpr int KSTEP = 32;  // K per instruction
  static constexpr int KPL = 8;     // K elements per lane
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  using TC = float;
  using frag = float;
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Fragment of a row-major M x K (or N x K) LDS array: lane l reads row row0 + l%16,
// K elements k0 + KPL*(l/16) .. +KPL.
template <typename M>
__device__ __forceinline__ typename M::frag frag_rows(const typename M::TC* base, int ld, int row0,
                                                      int k0, int lane) {
  return *reinterpret_cast<const typename M::frag*>(base + (row0 + (lane & 15)) * ld + k0 +
                                                    M::KPL * (lane >> 4));
}

// Fragment of an operand stored K x N (N contiguous): lane l needs column col0 + l%16,
// K elements k0 + KPL*(l/16) ..  Only used where KPL == 1 (fp32).
template <typename M>
__device__ __forceinline__ typename M::frag frag_cols(const typename M::TC* base, int ld, int k0,
                                                      int col0, int lane) {
  static_assert(M::KPL == 1, "strided fragment only for single-element lanes");
  return base[(k0 + (lane >> 4)) * ld + col0 + (lane & 15)];
}

// fp32 16x16x4 MFMA for the inverse's off-diagonal blocks (all paths).
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Byte layout of the workgroup's LDS.
template <typename Tin, int DK, int BV>
struct Smem {
  using TC = typename Mfma<Tin>::TC;
  static constexpr bool kBf16 = sizeof(TC) == 2;
  static constexpr int PADC = kBf16 ? 8 : 1;        // 16 B rows pad for bf16, 1 float for fp32
  static constexpr int LDK = DK + PADC;             // [64][DK] tiles and the [BV][DK] snapshot
  static constexpr int LDC = kChunk + PADC;         // [*][64] operand tiles
  static constexpr int LDF = kChunk + 1;            // fp32 [64][64] (A, inverse)
  static constexpr bool kKiT = kBf16;               // bf16 keeps Ki^T too (16 B fragments)
  static constexpr bool kXinT = !kBf16;             // fp32: inverse built in place in Tm
  static constexpr int CG = DK / 4, RG = kThreads / CG;

  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t oKg = 0;
  static constexpr size_t oQg = al(oKg + size_t(kChunk) * LDK * sizeof(TC));
  static constexpr size_t oKi = al(oQg + size_t(kChunk) * LDK * sizeof(TC));
  static constexpr size_t oKiT = al(oKi + size_t(kChunk) * LDK * sizeof(TC));
  static constexpr size_t oA = al(oKiT + (kKiT ? size_t(DK) * LDC * sizeof(TC) : 0));
  static constexpr size_t oX = al(oA + size_t(kChunk) * LDF * 4);
  static constexpr size_t oT = al(oX + (kXinT ? 0 : size_t(kChunk) * LDF * 4));
  static constexpr size_t oM = al(oT + size_t(kChunk) * LDC * sizeof(TC));
  static constexpr size_t oS = al(oM + size_t(kChunk) * LDC * sizeof(TC));
  static constexpr size_t scrCarry = size_t(RG) * DK * 4;
  static constexpr size_t scrY = size_t(4) * 16 * 17 * 4;
  static constexpr size_t oScr = al(oS + size_t(BV) * LDK * sizeof(TC));
  static constexpr size_t oBeta = al(oScr + (scrCarry > scrY ? scrCarry : scrY));
  static constexpr size_t oEgn = al(oBeta + kChunk * 4);
  static constexpr size_t kBytes = al(oEgn + DK * 4);
  // R^T and E^T ([BV][64]) reuse the A / inverse region, dead by then.
  static constexpr size_t oRT = oA;
  static constexpr size_t oET = al(oRT + size_t(BV) * LDC * sizeof(TC));
  static_assert(oET + size_t(BV) * LDC * sizeof(TC) <= oT, "R^T/E^T overflow their region");
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
  using L = Smem<Tin, DK, BV>;
  constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF;
  constexpr int CG = L::CG, RG = L::RG, RPG = kChunk / RG;
  constexpr int NVB = BV / 16;                 // 16-wide value blocks in the tile
  constexpr int NST = (DK / 16) * NVB / 4;     // S^T accumulator tiles per wave
  static_assert(NST >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::kBytes];
  TC* sKg = reinterpret_cast<TC*>(smem + L::oKg);
  TC* sQg = reinterpret_cast<TC*>(smem + L::oQg);
  TC* sKi = reinterpret_cast<TC*>(smem + L::oKi);
  TC* sKiT = reinterpret_cast<TC*>(smem + L::oKiT);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  TC* sT = reinterpret_cast<TC*>(smem + L::oT);
  float* sX = L::kXinT ? reinterpret_cast<float*>(smem + L::oT) : reinterpret_cast<float*>(smem + L::oX);
  constexpr int LDX = L::kXinT ? LDC : LDF;
  TC* sM = reinterpret_cast<TC*>(smem + L::oM);
  TC* sS = reinterpret_cast<TC*>(smem + L::oS);
  float* sScr = reinterpret_cast<float*>(smem + L::oScr);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
  float* sEgn = reinterpret_cast<float*>(smem + L::oEgn);
  TC* sRT = reinterpret_cast<TC*>(smem + L::oRT);
  TC* sET = reinterpret_cast<TC*>(smem + L::oET);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // ---- zero the operand tiles whose upper blocks are never written ---------------
  for (int i = tid; i < kChunk * LDC; i += kThreads) {
    sT[i] = from_f32<TC>(0.f);
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
#pragma unroll
    for (int i = 0; i < 4; ++i) sS[(16 * vb + lr) * LDK + kcol + i] = from_f32<TC>(sacc[s][i]);
  }

  const int cg = tid % CG, rg = tid / CG, j0 = 4 * cg;

  for (int64_t c0 = bos; c0 < eos; c0 += kChunk) {
    const int n = static_cast<int>((eos - c0) < kChunk ? (eos - c0) : kChunk);

    // ---- phase 1: prefix of g, exponentials, factor tiles --------------------------
    f32x4 gv[RPG], kv[RPG], qv[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = rg * RPG + i;
      if (r < n) {
        const int64_t off = ((c0 + r) * H + h) * DK + j0;
        gv[i] = *reinterpret_cast<const f32x4*>(g + off);
        kv[i] = load4(k + off);
        qv[i] = load4(q + off);
      } else {
        gv[i] = kv[i] = qv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // value tile in accumulator layout (row block = wave), for R = V - Kg S^T
    float vreg[NVB][4];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * lq + i;
        vreg[vb][i] = r < n ? to_f32(v[((c0 + r) * H + h) * DV + v0 + 16 * vb + lr]) : 0.f;
      }
    if (tid < kChunk) sBeta[tid] = tid < n ? beta[(c0 + tid) * H + h] : 0.f;

#pragma unroll
    for (int i = 1; i < RPG; ++i) gv[i] += gv[i - 1];
    *reinterpret_cast<f32x4*>(sScr + rg * DK + j0) = gv[RPG - 1];
    __syncthreads();
    f32x4 carry = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int r2 = 0; r2 < rg; ++r2) carry += *reinterpret_cast<const f32x4*>(sScr + r2 * DK + j0);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = rg * RPG + i;
      const f32x4 G = gv[i] + carry;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float eg = exp_hw(G[c]), ei = exp_hw(-G[c]);
        sKg[r * LDK + j0 + c] = from_f32<TC>(kv[i][c] * eg);
        sQg[r * LDK + j0 + c] = from_f32<TC>(scale * qv[i][c] * eg);
        const TC kic = from_f32<TC>(kv[i][c] * ei);
        sKi[r * LDK + j0 + c] = kic;
        if constexpr (L::kKiT) sKiT[(j0 + c) * LDC + r] = kic;
      }
    }
    if (rg == RG - 1) {
      const f32x4 G = gv[RPG - 1] + carry;
#pragma unroll
      for (int c = 0; c < 4; ++c) sEgn[j0 + c] = exp_hw(G[c]);
    }
    __syncthreads();

    // ---- phase 2: A = strict-lower(diag(beta) Kg Ki^T), M = lower(Qg Ki^T) --------
    {
      const bool isA = wave < 2;
      const TC* lhs = isA ? sKg : sQg;
      const int rbs[2] = {(wave & 1) ? 1 : 0, (wave & 1) ? 2 : 3};
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
        const int rb = rbs[pi];
        for (int cb = 0; cb <= rb; ++cb) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < DK; kk += M::KSTEP)
            acc = M::mma(frag_rows<M>(lhs, LDK, 16 * rb, kk, lane),
                         frag_rows<M>(sKi, LDK, 16 * cb, kk, lane), acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rb + 4 * lq + i, c = 16 * cb + lr;
            if (isA)
              sA[r * LDF + c] = c < r ? acc[i] * sBeta[r] : 0.f;
            else
              sM[r * LDC + c] = from_f32<TC>(c <= r ? acc[i] : 0.f);
          }
        }
      }
    }
    __syncthreads();

    // ---- phase 3: X = (I + A)^{-1}, then Tm = X diag(beta) ---------------------------
    // 3a: the four 16x16 unit-lower diagonal blocks, one wave, lane = (block, column).
    if (wave == 0) {
      const int bb = lane >> 4, c = lane & 15;
      const float* Ab = sA + (16 * bb) * LDF + 16 * bb;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < r; ++j) s -= Ab[r * LDF + j] * x[j];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sX[(16 * bb + r) * LDX + 16 * bb + c] = x[r];
    }
    __syncthreads();
    // 3b: off-diagonal blocks X_ij = -X_ii * sum_{k=j}^{i-1} A_ik X_kj, by distance i-j.
    {
      float* sY = sScr + wave * 16 * 17;
#pragma unroll
      for (int d = 1; d <= 3; ++d) {
        const bool active = wave < 4 - d;
        const int bi = wave + d, bj = wave;
        if (active) {
          f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int kb = bj; kb < bi; ++kb)
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4)
              y = mma_f32(sA[(16 * bi + lr) * LDF + 16 * kb + kk + lq],
                          sX[(16 * kb + kk + lq) * LDX + 16 * bj + lr], y);
#pragma unroll
          for (int i = 0; i < 4; ++i) sY[(4 * lq + i) * 17 + lr] = y[i];
        }
        __syncthreads();
        if (active) {
          f32x4 xij = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 16; kk += 4)
            xij = mma_f32(sX[(16 * bi + lr) * LDX + 16 * bi + kk + lq], sY[(kk + lq) * 17 + lr], xij);
#pragma unroll
          for (int i = 0; i < 4; ++i) sX[(16 * bi + 4 * lq + i) * LDX + 16 * bj + lr] = -xij[i];
        }
        __syncthreads();
      }
    }
    // Tm[r][c] = X[r][c] * beta_c (upper blocks stay zero)
    for (int idx = tid; idx < kChunk * kChunk; idx += kThreads) {
      const int r = idx >> 6, c = idx & 63;
      if (c <= r) {
        const float xv = sX[r * LDX + c];
        sT[r * LDC + c] = from_f32<TC>(xv * sBeta[c]);
      }
    }
    __syncthreads();

    // ---- phase 4a: P = Kg S^T, Qs = Qg S^T; R = V - P -> R^T -------------------------
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
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sRT[(16 * vb + lr) * LDC + 16 * wave + 4 * lq + i] = from_f32<TC>(vreg[vb][i] - accP[vb][i]);
    }
    __syncthreads();

    // ---- phase 4b: E = Tm R -> E^T ------------------------------------------------------
    {
      const int kend = 16 * (wave + 1);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < kend; kk += M::KSTEP)
          acc = M::mma(frag_rows<M>(sT, LDC, 16 * wave, kk, lane),
                       frag_rows<M>(sRT, LDC, 16 * vb, kk, lane), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) sET[(16 * vb + lr) * LDC + 16 * wave + 4 * lq + i] = from_f32<TC>(acc[i]);
      }
    }
    __syncthreads();

    // ---- phase 4c: O = Qs + M E (store); S^T = (S^T + Ki^T E) * e^{G_n} ---------------
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
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kc = 16 * kb + 4 * lq + i;
          acc[i] *= sEgn[kc];
          sS[(16 * vb + lr) * LDK + kc] = from_f32<TC>(acc[i]);
        }
        sacc[s] = acc;
      }
    }
    __syncthreads();
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
