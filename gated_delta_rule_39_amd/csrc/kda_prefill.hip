// Chunked KDA prefill on gfx950 (chunk = 64 tokens).
//
// Method: the per-token recurrence of "Kimi Delta Attention: The Linear Attention
// Behind Kimi K2 and Qwen3" (elsolitario.org, "How Kimi Delta Attention works step
// by step"), evaluated a chunk at a time; the state at the end of a chunk seeds the
// next ("Kimi Delta Attention Technical Deep Dive", "Systems and implementation
// tradeoffs" -> "Training").  The chunk algebra and the chunk-local tiles are
// described in kda_chunk.h; this file holds the two kernels built on them.
//
// Rows of the state S (the d_v index) never mix, so each (sequence, head) -- a
// "unit" -- is split into value tiles of BV rows that run as independent workgroups.
// The state tile is fp32 and lives in MFMA accumulators for the whole sequence,
// held transposed (S^T: rows = key channel) so that S^T <- (S^T + Ki^T E) Diag(e^{G_n})
// lands in the registers that hold it; after each chunk a snapshot (bf16 on the bf16
// path) goes to LDS as the next chunk's operand.
//
// prefill_kernel (fused): one workgroup per (unit, value tile) computes the chunk
//   tiles itself (ChunkProducer) and then the state step from LDS.  Every value tile
//   of a unit recomputes the same chunk tiles.  Used for fp32 inputs, and whenever
//   the producer/consumer kernel does not apply.
//
// prefill_coop_kernel (producer/consumer, bf16): per unit, NP producer workgroups
//   compute each chunk's tiles once (producer p takes chunks p, p+NP, ...) and
//   publish them into a ring of R slots in the caller's workspace, in MFMA fragment
//   order; NC consumer workgroups (value tiles) load the fragments straight into
//   registers, one chunk ahead, and run only the state step.  Hand-off: slots are
//   written and read with device-scope (sc1) accesses; a producer waits until all
//   its slot stores are acknowledged, then sets ready[slot] = chunk + 1 (a
//   device-scope atomic); consumers poll it, read the slot, and after using a chunk
//   add 1 to done[slot]; a producer reuses a slot only once all NC consumers are
//   done with its previous chunk.
//   Every wait is bounded: a wait that runs out, or sees the workspace's abort
//   word set, sets that word and the whole grid leaves its loops, so a broken
//   hand-off cannot hang the device (the results of such a call are invalid and the
//   abort word stays nonzero).  The grid (units x (NC + NP) <= compute units, one
//   workgroup per CU) is launched cooperatively, which guarantees that all its
//   workgroups are resident at once.  The workgroups of a unit are numbered so that
//   they run on one XCD (ids are dealt round-robin to the 8 XCDs) and the ring slots
//   they share stay in that XCD's L2.

#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {


__device__ __forceinline__ void unit_bounds(const PrefillArgs& a, int unit, int& n_seq, int& h,
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

// ====================================================================================
// Fused kernel
// ====================================================================================

template <typename Tin, int DK, int BV>
struct FusedLayout {
  using CL = ChunkLayout<Tin, DK>;
  using TC = typename CL::TC;
  static constexpr size_t oS = CL::kBytes;                           // [BV][LDK] snapshot
  static constexpr size_t kBytes = CL::al(oS + size_t(BV) * CL::LDK * sizeof(TC));
  // R'^T and E^T ([BV][64]) reuse the A (and inverse) region, dead by then.
  static constexpr size_t oRT = CL::oA;
  static constexpr size_t oET = CL::al(oRT + size_t(BV) * CL::LDC * sizeof(TC));
  static_assert(oET + size_t(BV) * CL::LDC * sizeof(TC) <= CL::oScr, "R^T/E^T overflow");
  static_assert(kBytes <= 160 * 1024, "LDS budget exceeded");
};

template <typename Tin, int DK, int BV>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
  using CP = ChunkProducer<Tin, DK>;
  using M = typename CP::M;
  using TC = typename CP::TC;
  using FL = FusedLayout<Tin, DK, BV>;
  using ST = StateTiles<DK, BV>;
  constexpr int LDK = CP::LDK, LDC = CP::LDC;
  constexpr int NVB = BV / 16;

  __shared__ __attribute__((aligned(16))) unsigned char smem[FL::kBytes];
  TC* sS = reinterpret_cast<TC*>(smem + FL::oS);
  TC* sRT = reinterpret_cast<TC*>(smem + FL::oRT);
  TC* sET = reinterpret_cast<TC*>(smem + FL::oET);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lr = lane & 15, lq = lane >> 4;

  int unit, vt, n_seq, h;
  int64_t bos, eos;
  unit_role(blockIdx.x, a.NV, a.units, a.xcd_remap, unit, vt);
  unit_bounds(a, unit, n_seq, h, bos, eos);
  const int v0 = vt * BV;
  const Tin* v = static_cast<const Tin*>(a.v);
  Tin* o = static_cast<Tin*>(a.o);

  CP cp;
  cp.init(smem, static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), a.g, a.beta, a.H, h,
          a.scale, tid, wave);
  f32x4 sacc[ST::NST];
  const int64_t st_base = (static_cast<int64_t>(n_seq) * a.H + h) * a.DV * DK;
  load_state<DK, BV, LDK>(sacc, a.initial_state, st_base, v0, sS, wave, lane);

  ValueRegs<Tin, NVB> vr;
  if (bos < eos) {
    const int n0 = static_cast<int>(min(eos - bos, static_cast<int64_t>(kChunk)));
    cp.load(bos, n0);
    vr.load(v, bos, n0, a.H, h, a.DV, v0, wave, lane);
  }

  for (int64_t c0 = bos; c0 < eos; c0 += kChunk) {
    const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
    const int64_t c1 = c0 + kChunk;
    const bool has_next = c1 < eos;
    const int n1 = has_next ? static_cast<int>(min(eos - c1, static_cast<int64_t>(kChunk))) : 0;

    cp.factors(n, has_next, c1, n1);
    cp.products();
    cp.inverse();

    // ---- P = Kg S^T, Qs = Qg S^T; R' = diag(beta)(V - P) -> R'^T ---------------------
    f32x4 accQ[NVB];
    {
      f32x4 accP[NVB];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) accP[vb] = accQ[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < DK; kk += M::KSTEP) {
        const auto aK = frag_rows<M>(cp.sKg, LDK, 16 * wave, kk, lane);
        const auto aQ = frag_rows<M>(cp.sQg, LDK, 16 * wave, kk, lane);
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const auto bS = frag_rows<M>(sS, LDK, 16 * vb, kk, lane);
          accP[vb] = M::mma(aK, bS, accP[vb]);
          accQ[vb] = M::mma(aQ, bS, accQ[vb]);
        }
      }
      const f32x4 bt = *reinterpret_cast<const f32x4*>(cp.sBeta + 16 * wave + 4 * lq);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 rv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = 16 * wave + 4 * lq + i < n;
          rv[i] = ok ? bt[i] * (vr.f32(vb, i) - accP[vb][i]) : 0.f;
        }
        store4(sRT + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, rv);
      }
      // the value registers are free: load the next chunk's tile
      if (has_next) vr.load(v, c1, n1, a.H, h, a.DV, v0, wave, lane);
    }
    lds_barrier();

    // ---- E = X R' -> E^T ---------------------------------------------------------------
    {
      const int kend = 16 * (wave + 1);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < kend; kk += M::KSTEP)
          acc = M::mma(frag_rows<M>(cp.sTm, LDC, 16 * wave, kk, lane),
                       frag_rows<M>(sRT, LDC, 16 * vb, kk, lane), acc);
        store4(sET + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, acc);
      }
    }
    lds_barrier();

    // ---- O = Qs + M E (store); S^T = (S^T + Ki^T E) Diag(e^{G_n}) -----------------------
    {
      const int kend = 16 * (wave + 1);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 acc = accQ[vb];
        for (int kk = 0; kk < kend; kk += M::KSTEP)
          acc = M::mma(frag_rows<M>(cp.sM, LDC, 16 * wave, kk, lane),
                       frag_rows<M>(sET, LDC, 16 * vb, kk, lane), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * wave + 4 * lq + i;
          if (r < n) o[((c0 + r) * a.H + h) * a.DV + v0 + 16 * vb + lr] = from_f32<Tin>(acc[i]);
        }
      }
#pragma unroll
      for (int s = 0; s < ST::NST; ++s) {
        const int kb = ST::kb(wave, s), vb = ST::vb(s);
        f32x4 acc = sacc[s];
#pragma unroll
        for (int kk = 0; kk < kChunk; kk += M::KSTEP) {
          typename M::frag af;
          if constexpr (CP::L::kKiT)
            af = frag_rows<M>(cp.sKiT, LDC, 16 * kb, kk, lane);
          else
            af = frag_cols<M>(cp.sKi, LDK, kk, 16 * kb, lane);
          acc = M::mma(af, frag_rows<M>(sET, LDC, 16 * vb, kk, lane), acc);
        }
        const f32x4 e = *reinterpret_cast<const f32x4*>(cp.sEgn + 16 * kb + 4 * lq);
        acc *= e;
        store4(sS + (16 * vb + lr) * LDK + 16 * kb + 4 * lq, acc);
        sacc[s] = acc;
      }
    }
    lds_barrier();
  }

  if (a.final_state) store_state<DK, BV>(sacc, a.final_state, st_base, v0, wave, lane);
}

// ====================================================================================
// Producer / consumer kernel (bf16)
// ====================================================================================

// One ring slot: the chunk's operands in MFMA fragment order.  A fragment block is
// the 16 bytes each of the 64 lanes loads for one 16x32 operand step (1 KiB), so a
// consumer wave reads every block as one contiguous 1 KiB load.
template <int DK>
struct SlotLayout {
  static constexpr int kKs = DK / 32;                 // k steps of Kg / Qg
  static constexpr int nKg = 4 * kKs;                 // (row block, k step)
  static constexpr int nKiT = (DK / 16) * 2;          // (key block, token step)
  static constexpr int nTm = 8;                       // (row block, token step)
  static constexpr size_t kFrag = 1024;
  static constexpr size_t oKg = 0;
  static constexpr size_t oQg = oKg + nKg * kFrag;
  static constexpr size_t oKiT = oQg + nKg * kFrag;
  static constexpr size_t oTm = oKiT + nKiT * kFrag;
  static constexpr size_t oM = oTm + nTm * kFrag;
  static constexpr size_t oBeta = oM + nTm * kFrag;   // 64 fp32
  static constexpr size_t oEgn = oBeta + 64 * 4;      // DK fp32
  static constexpr size_t kBytes = (oEgn + DK * 4 + 255) & ~size_t(255);
  static constexpr int nBlocks = 2 * nKg + nKiT + 2 * nTm;
};

// Workspace: [0, 256) header (word 0: abort), then per-unit flags ready[R], done[R]
// (int32), then the ring slots.
constexpr size_t kWsHeader = 256;
__host__ __device__ inline size_t coop_flags_bytes(int units, int R) {
  return (size_t(units) * 2 * R * 4 + 255) & ~size_t(255);
}
template <int DK>
__host__ __device__ inline size_t coop_workspace_bytes(int units, int R) {
  return kWsHeader + coop_flags_bytes(units, R) + size_t(units) * R * SlotLayout<DK>::kBytes;
}

constexpr uint32_t kSpinLimit = 1u << 22;   // ~ a second of s_sleep polling

// Ring slots are written and read with device-scope (sc1) buffer accesses: a store
// is acknowledged only once it is visible device-wide and a load reads the
// device-coherent copy, so the hand-off needs no cache write-back or invalidate.
constexpr int kDeviceScope = 16;             // cache-policy bit SC1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(unsigned char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void ring_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16x8 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ void ring_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ bf16x8 ring_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope);
  return __builtin_bit_cast(bf16x8, x);
}
__device__ __forceinline__ f32x4 ring_load16f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope);
  return __builtin_bit_cast(f32x4, x);
}

// Wait (one lane) until *p >= target.  False if the wait ran out or the grid aborted;
// a wait that runs out raises the abort word.
__device__ __forceinline__ bool wait_at_least(const int* p, int target, int* abort_word) {
  for (uint32_t it = 0;; ++it) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    if ((it & 15) == 15 &&
        __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
      return false;
    if (it >= kSpinLimit) {
      __hip_atomic_store(abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

template <int DK, int BV>
struct ConsumerLayout {
  static constexpr int LDK = DK + 8, LDC = kChunk + 8;
  static constexpr size_t oS = 0;                                         // [BV][LDK] bf16
  static constexpr size_t oRT = (oS + size_t(BV) * LDK * 2 + 15) & ~size_t(15);   // [BV][LDC]
  static constexpr size_t oET = (oRT + size_t(BV) * LDC * 2 + 15) & ~size_t(15);
  static constexpr size_t oFlag = (oET + size_t(BV) * LDC * 2 + 15) & ~size_t(15);
  static constexpr size_t kBytes = oFlag + 16;
};

// A consumer's operand fragments for one chunk (wave w: row block w; key blocks of
// its state tiles).
template <int DK>
struct ChunkFrags {
  using SL = SlotLayout<DK>;
  static constexpr int KPW = DK / 64;
  bf16x8 kg[SL::kKs], qg[SL::kKs], tm[2], mm[2], kit[KPW][2];
  f32x4 bt;          // beta of rows 16w + 4*lq .. +3
  f32x4 egn[KPW];    // e^{G_n} of key channels 16*kb + 4*lq .. +3
  // slot: byte offset of the slot in the unit's ring
  __device__ __forceinline__ void load_kq(__amdgpu_buffer_rsrc_t r, uint32_t slot, int wave,
                                          int lane) {
#pragma unroll
    for (int s = 0; s < SL::kKs; ++s) {
      kg[s] = ring_load16(r, slot + SL::oKg + (wave * SL::kKs + s) * SL::kFrag + 16 * lane);
      qg[s] = ring_load16(r, slot + SL::oQg + (wave * SL::kKs + s) * SL::kFrag + 16 * lane);
    }
    bt = ring_load16f(r, slot + SL::oBeta + (16 * wave + 4 * (lane >> 4)) * 4);
  }
  __device__ __forceinline__ void load_tm(__amdgpu_buffer_rsrc_t r, uint32_t slot, int wave,
                                          int lane) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      tm[t] = ring_load16(r, slot + SL::oTm + (wave * 2 + t) * SL::kFrag + 16 * lane);
  }
  __device__ __forceinline__ void load_rest(__amdgpu_buffer_rsrc_t r, uint32_t slot, int wave,
                                            int lane) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      mm[t] = ring_load16(r, slot + SL::oM + (wave * 2 + t) * SL::kFrag + 16 * lane);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int kb = wave * KPW + j;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        kit[j][t] = ring_load16(r, slot + SL::oKiT + (kb * 2 + t) * SL::kFrag + 16 * lane);
      egn[j] = ring_load16f(r, slot + SL::oEgn + (16 * kb + 4 * (lane >> 4)) * 4);
    }
  }
};

template <int DK, int BV>
struct CoopLayout {
  static constexpr size_t a = ChunkLayout<bf16, DK>::kBytes;
  static constexpr size_t b = ConsumerLayout<DK, BV>::kBytes;
  static constexpr size_t kBytes = a > b ? a : b;
  static_assert(kBytes <= 160 * 1024, "LDS budget exceeded");
};

template <int DK, int BV>
__global__ __launch_bounds__(kThreads, 1) void prefill_coop_kernel(PrefillArgs a) {
  using CP = ChunkProducer<bf16, DK>;
  using M = Mfma<bf16>;
  using SL = SlotLayout<DK>;
  using CL = ConsumerLayout<DK, BV>;
  using ST = StateTiles<DK, BV>;
  constexpr int NVB = BV / 16;
  constexpr int LDK = CL::LDK, LDC = CL::LDC;

  __shared__ __attribute__((aligned(16))) unsigned char smem[CoopLayout<DK, BV>::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  const int W = a.NC + a.NP;
  int unit, role, n_seq, h;
  int64_t bos, eos;
  unit_role(blockIdx.x, W, a.units, a.xcd_remap, unit, role);
  unit_bounds(a, unit, n_seq, h, bos, eos);
  const int nch = static_cast<int>((eos - bos + kChunk - 1) / kChunk);

  int* abort_word = reinterpret_cast<int*>(a.workspace);
  int* ready = reinterpret_cast<int*>(a.workspace + kWsHeader) + size_t(unit) * 2 * a.R;
  int* done = ready + a.R;
  unsigned char* ring = a.workspace + kWsHeader + coop_flags_bytes(a.units, a.R) +
                        size_t(unit) * a.R * SL::kBytes;
  int* sFlag = reinterpret_cast<int*>(smem + CL::oFlag);   // consumer: wait result
  const __amdgpu_buffer_rsrc_t rr = ring_rsrc(ring, static_cast<uint32_t>(a.R * SL::kBytes));

  if (role >= a.NC) {
    // ================================ producer ==================================
    const int p = role - a.NC;
    CP cp;
    cp.init(smem, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), a.g, a.beta,
            a.H, h, a.scale, tid, wave);
    if (p < nch) {
      const int64_t c0 = bos + int64_t(p) * kChunk;
      cp.load(c0, static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk))));
    }
    int* pFlag = reinterpret_cast<int*>(smem + ChunkLayout<bf16, DK>::oScr);
    for (int c = p; c < nch; c += a.NP) {
      const int64_t c0 = bos + int64_t(c) * kChunk;
      const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
      const int cn = c + a.NP;
      const bool has_next = cn < nch;
      const int64_t c1 = bos + int64_t(cn) * kChunk;
      const int n1 = has_next ? static_cast<int>(min(eos - c1, static_cast<int64_t>(kChunk))) : 0;
      cp.factors(n, has_next, c1, n1);
      cp.products();
      cp.inverse();
      // the slot must have been read by every consumer of its previous chunk
      const int s = c % a.R;
      if (tid == 0) pFlag[0] = wait_at_least(done + s, a.NC * (c / a.R), abort_word) ? 1 : 0;
      lds_barrier();
      const bool ok = pFlag[0] != 0;
      lds_barrier();
      if (!ok) break;
      const uint32_t slot = static_cast<uint32_t>(s) * SL::kBytes;
      // fragment blocks: waves take blocks w, w+4, ...
      for (int b = wave; b < SL::nBlocks; b += 4) {
        bf16x8 f;
        uint32_t off;
        if (b < SL::nKg) {
          f = frag_rows<M>(cp.sKg, CP::LDK, 16 * (b / SL::kKs), 32 * (b % SL::kKs), lane);
          off = SL::oKg + b * SL::kFrag;
        } else if (b < 2 * SL::nKg) {
          const int i = b - SL::nKg;
          f = frag_rows<M>(cp.sQg, CP::LDK, 16 * (i / SL::kKs), 32 * (i % SL::kKs), lane);
          off = SL::oQg + i * SL::kFrag;
        } else if (b < 2 * SL::nKg + SL::nKiT) {
          const int i = b - 2 * SL::nKg;
          f = frag_rows<M>(cp.sKiT, CP::LDC, 16 * (i / 2), 32 * (i % 2), lane);
          off = SL::oKiT + i * SL::kFrag;
        } else if (b < 2 * SL::nKg + SL::nKiT + SL::nTm) {
          const int i = b - 2 * SL::nKg - SL::nKiT;
          f = frag_rows<M>(cp.sTm, CP::LDC, 16 * (i / 2), 32 * (i % 2), lane);
          off = SL::oTm + i * SL::kFrag;
        } else {
          const int i = b - 2 * SL::nKg - SL::nKiT - SL::nTm;
          f = frag_rows<M>(cp.sM, CP::LDC, 16 * (i / 2), 32 * (i % 2), lane);
          off = SL::oM + i * SL::kFrag;
        }
        ring_store16(rr, slot + off + 16 * lane, f);
      }
      if (tid < kChunk) ring_store4(rr, slot + SL::oBeta + 4 * tid, cp.sBeta[tid]);
      if (tid < DK) ring_store4(rr, slot + SL::oEgn + 4 * tid, cp.sEgn[tid]);
      // every store of the workgroup acknowledged (device-visible), then publish
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
      if (tid == 0) __hip_atomic_store(ready + s, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // ================================== consumer =====================================
  const int vt = role;
  const int v0 = vt * BV;
  bf16* sS = reinterpret_cast<bf16*>(smem + CL::oS);
  bf16* sRT = reinterpret_cast<bf16*>(smem + CL::oRT);
  bf16* sET = reinterpret_cast<bf16*>(smem + CL::oET);
  const bf16* v = static_cast<const bf16*>(a.v);
  bf16* o = static_cast<bf16*>(a.o);

  f32x4 sacc[ST::NST];
  const int64_t st_base = (static_cast<int64_t>(n_seq) * a.H + h) * a.DV * DK;
  load_state<DK, BV, LDK>(sacc, a.initial_state, st_base, v0, sS, wave, lane);

  ChunkFrags<DK> fr;
  ValueRegs<bf16, NVB> vr;
  bool ok = true;
  if (nch > 0) {
    if (tid == 0) sFlag[0] = wait_at_least(ready, 1, abort_word) ? 1 : 0;
    lds_barrier();
    ok = sFlag[0] != 0;
    if (ok) {
      fr.load_kq(rr, 0, wave, lane);
      fr.load_tm(rr, 0, wave, lane);
      fr.load_rest(rr, 0, wave, lane);
      vr.load(v, bos, static_cast<int>(min(eos - bos, static_cast<int64_t>(kChunk))), a.H, h,
              a.DV, v0, wave, lane);
    }
  }

  for (int c = 0; ok && c < nch; ++c) {
    const int64_t c0 = bos + int64_t(c) * kChunk;
    const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
    const bool has_next = c + 1 < nch;
    const int64_t c1 = c0 + kChunk;
    const int n1 = has_next ? static_cast<int>(min(eos - c1, static_cast<int64_t>(kChunk))) : 0;
    const uint32_t nslot = static_cast<uint32_t>((c + 1) % a.R) * SL::kBytes;
    // wait for the next chunk's slot while this chunk computes
    if (tid == 0 && has_next)
      sFlag[1] = wait_at_least(ready + (c + 1) % a.R, c + 2, abort_word) ? 1 : 0;

    // ---- P = Kg S^T, Qs = Qg S^T; R' = diag(beta)(V - P) -> R'^T ---------------------
    f32x4 accQ[NVB];
    {
      f32x4 accP[NVB];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) accP[vb] = accQ[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < SL::kKs; ++ks) {
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const auto bS = frag_rows<M>(sS, LDK, 16 * vb, 32 * ks, lane);
          accP[vb] = M::mma(fr.kg[ks], bS, accP[vb]);
          accQ[vb] = M::mma(fr.qg[ks], bS, accQ[vb]);
        }
      }
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f32x4 rv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool okr = 16 * wave + 4 * lq + i < n;
          rv[i] = okr ? fr.bt[i] * (vr.f32(vb, i) - accP[vb][i]) : 0.f;
        }
        store4(sRT + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, rv);
      }
    }
    lds_barrier();
    const bool nok = has_next ? sFlag[1] != 0 : true;
    if (has_next && nok) {
      fr.load_kq(rr, nslot, wave, lane);
      vr.load(v, c1, n1, a.H, h, a.DV, v0, wave, lane);
    }

    // ---- E = X R' -> E^T ---------------------------------------------------------------
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      acc = M::mma(fr.tm[0], frag_rows<M>(sRT, LDC, 16 * vb, 0, lane), acc);
      if (wave >= 2) acc = M::mma(fr.tm[1], frag_rows<M>(sRT, LDC, 16 * vb, 32, lane), acc);
      store4(sET + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, acc);
    }
    lds_barrier();
    if (has_next && nok) fr.load_tm(rr, nslot, wave, lane);

    // ---- O = Qs + M E (store); S^T = (S^T + Ki^T E) Diag(e^{G_n}) -----------------------
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 acc = accQ[vb];
      acc = M::mma(fr.mm[0], frag_rows<M>(sET, LDC, 16 * vb, 0, lane), acc);
      if (wave >= 2) acc = M::mma(fr.mm[1], frag_rows<M>(sET, LDC, 16 * vb, 32, lane), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * lq + i;
        if (r < n) o[((c0 + r) * a.H + h) * a.DV + v0 + 16 * vb + lr] = from_f32<bf16>(acc[i]);
      }
    }
#pragma unroll
    for (int s = 0; s < ST::NST; ++s) {
      const int j = s / NVB, vb = ST::vb(s);
      const int kb = ST::kb(wave, s);
      f32x4 acc = sacc[s];
      acc = M::mma(fr.kit[j][0], frag_rows<M>(sET, LDC, 16 * vb, 0, lane), acc);
      acc = M::mma(fr.kit[j][1], frag_rows<M>(sET, LDC, 16 * vb, 32, lane), acc);
      acc *= fr.egn[j];
      store4(sS + (16 * vb + lr) * LDK + 16 * kb + 4 * lq, acc);
      sacc[s] = acc;
    }
    if (has_next && nok) fr.load_rest(rr, nslot, wave, lane);
    lds_barrier();
    // this chunk's fragments were all used: free its slot
    if (tid == 0) __hip_atomic_fetch_add(done + c % a.R, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = nok;
  }

  if (ok && a.final_state) store_state<DK, BV>(sacc, a.final_state, st_base, v0, wave, lane);
}

// Zero the abort word and the hand-off flags before a producer/consumer launch.
__global__ void coop_reset_kernel(int* words, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    words[i] = 0;
}

// ====================================================================================
// Launch
// ====================================================================================

// Largest value-tile height each dtype / d_k instantiation of the fused kernel
// supports (LDS budget: fp32 operands are twice the size of bf16 ones).
constexpr int max_bv(bool fp32, int dk) { return fp32 ? (dk == 128 ? 16 : 32) : 64; }
int prefill_max_bv(int dtype, int dk) { return max_bv(dtype == 0, dk); }

template <typename Tin, int DK>
static hipError_t launch_fused_dk(int bv, const PrefillArgs& a, hipStream_t stream) {
  constexpr int kMax = max_bv(sizeof(Tin) == 4, DK);
  const dim3 grid(a.units * a.NV), block(kThreads);
  if constexpr (kMax >= 64) {
    if (bv == 64) {
      hipLaunchKernelGGL((prefill_kernel<Tin, DK, 64>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if constexpr (kMax >= 32) {
    if (bv == 32) {
      hipLaunchKernelGGL((prefill_kernel<Tin, DK, 32>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_kernel<Tin, DK, 16>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Fused kernel.  bv in {16, 32, 64}, bv <= prefill_max_bv; a.NV = DV / bv.
hipError_t launch_prefill(int dtype, int dk, int bv, const PrefillArgs& a, hipStream_t stream) {
  if (dtype == 1)
    return dk == 64 ? launch_fused_dk<bf16, 64>(bv, a, stream)
                    : launch_fused_dk<bf16, 128>(bv, a, stream);
  return dk == 64 ? launch_fused_dk<float, 64>(bv, a, stream)
                  : launch_fused_dk<float, 128>(bv, a, stream);
}

size_t prefill_coop_workspace_bytes(int dk, int units, int R) {
  return dk == 64 ? coop_workspace_bytes<64>(units, R) : coop_workspace_bytes<128>(units, R);
}

template <int DK, int BV>
static hipError_t launch_coop_t(const PrefillArgs& a, hipStream_t stream) {
  const int nwords = static_cast<int>((kWsHeader + coop_flags_bytes(a.units, a.R)) / 4);
  hipLaunchKernelGGL(coop_reset_kernel, dim3((nwords + 255) / 256), dim3(256), 0, stream,
                     reinterpret_cast<int*>(a.workspace), nwords);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&prefill_coop_kernel<DK, BV>),
                                    dim3(a.units * (a.NC + a.NP)), dim3(kThreads), params, 0,
                                    stream);
}

// Producer/consumer kernel (bf16).  a.NC consumers of a.DV / a.NC rows, a.NP producers,
// a.R ring slots per unit; a.workspace holds prefill_coop_workspace_bytes bytes.
hipError_t launch_prefill_coop(int dk, const PrefillArgs& a, hipStream_t stream) {
  const int bv = a.DV / a.NC;
  if (dk == 64) {
    if (bv == 64) return launch_coop_t<64, 64>(a, stream);
    if (bv == 32) return launch_coop_t<64, 32>(a, stream);
    return launch_coop_t<64, 16>(a, stream);
  }
  if (bv == 128) return launch_coop_t<128, 128>(a, stream);
  if (bv == 64) return launch_coop_t<128, 64>(a, stream);
  if (bv == 32) return launch_coop_t<128, 32>(a, stream);
  return launch_coop_t<128, 16>(a, stream);
}

}  // namespace kda
