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

#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "kda_chunk.h"
#include "kda_launch.h"
#include "kda_tiles.h"
#include "kda_wy.h"

namespace kda {

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

// DECAY: 0 = g per key channel (KDA), 1 = one g per token and head (Gated DeltaNet),
// 2 = no decay (DeltaNet).  Only the gate loads differ.
// STATES (the backward's forward sweep): instead of o, write the state at the start of
// every chunk, bf16, to a.chunk_states as [slot][H][d_v][d_k] with
// slot = chunk_slot_base(sequence) + chunk index (kda_tiles.h).
template <typename Tin, int DK, int BV, int DECAY, bool STATES = false>
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
          a.scale, tid, wave, a.flags);
  f32x4 sacc[ST::NST];
  const int64_t st_base = (static_cast<int64_t>(n_seq) * a.H + h) * a.DV * DK;
  load_state<DK, BV, LDK>(sacc, a.initial_state, st_base, v0, sS, wave, lane);

  ValueRegs<Tin, NVB> vr;
  if (bos < eos) {
    const int n0 = static_cast<int>(min(eos - bos, static_cast<int64_t>(kChunk)));
    cp.template load<DECAY>(bos, n0);
    vr.load(v, bos, n0, a.H, h, a.DV, v0, wave, lane);
  }

  for (int64_t c0 = bos; c0 < eos; c0 += kChunk) {
    const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
    const int64_t c1 = c0 + kChunk;
    const bool has_next = c1 < eos;
    const int n1 = has_next ? static_cast<int>(min(eos - c1, static_cast<int64_t>(kChunk))) : 0;
    if constexpr (STATES) {
      const int64_t slot = chunk_slot_base(n_seq, bos) + (c0 - bos) / kChunk;
      store_state_bf16<DK, BV>(sacc, static_cast<bf16*>(a.chunk_states),
                               ((slot * a.H + h) * a.DV) * DK, v0, wave, lane);
    }

    cp.template factors<DECAY>(n, has_next, c1, n1);
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
        if constexpr (!STATES) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * wave + 4 * lq + i;
            if (r < n) o[((c0 + r) * a.H + h) * a.DV + v0 + 16 * vb + lr] = from_f32<Tin>(acc[i]);
          }
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
// Producer / consumer kernel (bf16, WY form; the algebra is in kda_wy.h)
// ====================================================================================

// Workspace: [0, 256) header (word 0: this call aborted; word 1: some call aborted
// since the caller last cleared it -- the launch's reset kernel clears word 0 and the
// flags, never word 1), then per-unit flags ready[R], done[R], arrive, pad (int32),
// then the ring slots.
// With a lane plan, the header is followed by it: lane_off[lanes + 1], lane_units[units]
// and each lane's total chunk count lane_tot[lanes] (int32), written by coop_prep_kernel.
constexpr size_t kWsHeader = 256;
__host__ __device__ inline int coop_flag_words(int R) { return 2 * R + 2; }
__host__ __device__ inline size_t coop_flags_bytes(int lanes, int R) {
  return (size_t(lanes) * coop_flag_words(R) * 4 + 255) & ~size_t(255);
}
__host__ __device__ inline size_t coop_plan_bytes(int lanes, int units, bool plan) {
  return plan ? (size_t(2 * lanes + 1 + units) * 4 + 255) & ~size_t(255) : 0;
}
__device__ __forceinline__ size_t coop_plan_bytes(const PrefillArgs& a) {
  return coop_plan_bytes(a.lanes, a.units, a.lane_units != nullptr);
}

// s_getreg operand for the XCC_ID hardware register (id 20, bits 0..15): the XCD the
// wave runs on.
constexpr int kHwRegXccId = 20 | (0 << 6) | (15 << 11);
template <int DK, int DV>
__host__ __device__ inline size_t coop_workspace_bytes(int lanes, int units, int R, bool plan) {
  return kWsHeader + coop_plan_bytes(lanes, units, plan) + coop_flags_bytes(lanes, R) +
         size_t(lanes) * R * WySlot<DK, DV>::kBytes;
}

constexpr uint32_t kSpinLimit = 1u << 22;   // ~ a second of s_sleep polling

// Raise the abort: word 0 (this call; every waiting workgroup then leaves its loop)
// and the sticky word 1.
__device__ __forceinline__ void raise_abort(int* abort_word) {
  __hip_atomic_store(abort_word + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- phase clock (only in a build with -DKDA_PHASE_STAMPS) ---------------------------
// Each producer/consumer workgroup sums s_memtime ticks per phase of its chunk loop (the
// phases are the stretches between mark(i - 1) and mark(i)) and writes the sums, its
// chunk count and its role when it leaves; kda_phase_read() copies them out.  The
// product build compiles none of it (KDA_PHASE, kda_device.h, expands to nothing).
#if defined(KDA_PHASE_STAMPS)
constexpr int kPhaseWgs = 4096, kPhaseWords = 16;
__device__ unsigned int g_phase[kPhaseWgs * kPhaseWords];
struct PhaseClock {
  unsigned long long t[10];
  unsigned acc[10];
  int chunks;
  __device__ __forceinline__ void start() {
    for (int i = 0; i < 10; ++i) acc[i] = 0;
    chunks = 0;
  }
  __device__ __forceinline__ void mark(int i) { t[i] = __builtin_amdgcn_s_memtime(); }
  __device__ __forceinline__ void close(int n) {
    for (int i = 1; i < n; ++i) acc[i] += static_cast<unsigned>(t[i] - t[i - 1]);
    ++chunks;
  }
  __device__ __forceinline__ void write(int tid, int role) const {
    if (tid != 0 || blockIdx.x >= kPhaseWgs) return;
    unsigned int* w = g_phase + blockIdx.x * kPhaseWords;
    for (int i = 0; i < 10; ++i) w[i] = acc[i];
    w[14] = static_cast<unsigned>(chunks);
    w[15] = static_cast<unsigned>(role);
  }
};
#endif

// Wait (one lane) until *p >= target.  False if the wait ran out or the grid aborted;
// a wait that runs out raises the abort word.
__device__ __forceinline__ bool wait_at_least(const int* p, int target, int* abort_word) {
  for (uint32_t it = 0;; ++it) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    if ((it & 15) == 15 &&
        __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
      return false;
    if (it >= kSpinLimit) {
      raise_abort(abort_word);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Barrier after this wave's global accesses have completed (loads landed, LDS
// copies written, stores acknowledged) and its LDS operations are done.
__device__ __forceinline__ void vm_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A consumer whose hand-off aborted leaves its outputs invalid.  Make that visible
// instead of leaving stale values: NaN in every element it owns -- value columns
// [v0, v0 + ncols) of the unit's o rows, of its final state and (STATES) of its
// chunk-start states.
template <int DK, int DV, bool STATES>
__device__ __forceinline__ void poison_outputs(const PrefillArgs& a, int n_seq, int h, int64_t bos,
                                            int64_t eos, int nch, int v0, int ncols, int tid) {
  const int vpr = ncols / 8;   // 16-byte vectors per row
  const u32x4 nan2 = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
  const u32x4 nan4 = u32x4{0x7fc00000u, 0x7fc00000u, 0x7fc00000u, 0x7fc00000u};
  if (a.o) {
    bf16* o = static_cast<bf16*>(a.o);
    for (int64_t i = tid; i < (eos - bos) * vpr; i += kThreads) {
      const int64_t r = bos + i / vpr;
      *reinterpret_cast<u32x4*>(o + (r * a.H + h) * DV + v0 + 8 * (i % vpr)) = nan2;
    }
  }
  const int64_t st_base = (static_cast<int64_t>(n_seq) * a.H + h) * DV * DK;
  if (a.final_state)
    for (int i = tid; i < ncols * DK / 4; i += kThreads)
      *reinterpret_cast<u32x4*>(a.final_state + st_base + int64_t(v0) * DK + 4 * i) = nan4;
  if constexpr (STATES) {
    bf16* cs = static_cast<bf16*>(a.chunk_states);
    const int64_t slot0 = chunk_slot_base(n_seq, bos);
    for (int64_t i = tid; i < int64_t(nch) * ncols * DK / 8; i += kThreads) {
      const int64_t c = i / (ncols * DK / 8), e = i % (ncols * DK / 8);
      *reinterpret_cast<u32x4*>(cs + ((slot0 + c) * a.H + h) * DV * DK + int64_t(v0) * DK +
                                8 * e) = nan2;
    }
  }
}

// Consumer LDS: two staging buffers, two output tiles [64][BV + 8] bf16, flags.
template <int DK, int DV>
struct WyConsumerLayout {
  static constexpr int LDO = 128 + 8;   // output tile row (the widest value tile)
  static constexpr size_t oStage = 0;
  static constexpr size_t oO = 2 * WySlot<DK, DV>::kStage;
  static constexpr size_t kOBytes = size_t(kChunk) * LDO * 2;
  static constexpr size_t oFlag = oO + 2 * kOBytes;
  static constexpr size_t kBytes = oFlag + 16;
};

// Split consumer LDS: the bf16 S^T operand fragments [KS][4] (1 KiB each), the bf16 E
// operand fragments [2][4], two output tiles [64][64 + 8] bf16 (chunk g's in tile g % 2),
// flags.
struct WySplitLayout {
  static constexpr int NVT = 4;                 // 64 value columns per consumer
  static constexpr int LDO = 16 * NVT + 8;
  static constexpr size_t oSb = 0;
  static constexpr size_t oEb = oSb + size_t(4) * NVT * 1024;
  static constexpr size_t oO = oEb + size_t(2) * NVT * 1024;
  static constexpr size_t kOBytes = size_t(kChunk) * LDO * 2;
  static constexpr size_t oFlag = oO + 2 * kOBytes;
  static constexpr size_t kBytes = oFlag + 16;
};

// ---- lanes ---------------------------------------------------------------------------
// A lane is one set of NC consumer and NP producer workgroups.  It processes a list of
// units one after another: its chunk stream is the concatenation of their chunks, and the
// ring slots, flags and producer stripes run over that stream (global chunk index g).
// Without a lane plan (a.lane_units == nullptr) lane l is unit l.
struct LaneUnit {
  int unit, n_seq, h;
  int64_t bos, eos;
  int nch, g0;   // chunks of the unit; index of its first chunk in the lane's stream
};
__device__ __forceinline__ int lane_count(const PrefillArgs& a, int lid) {
  return a.lane_units ? a.lane_off[lid + 1] - a.lane_off[lid] : 1;
}
__device__ __forceinline__ void lane_unit(const PrefillArgs& a, int lid, int i, int g0,
                                          LaneUnit& u) {
  u.unit = a.lane_units ? a.lane_units[a.lane_off[lid] + i] : lid;
  unit_bounds(a, u.unit, u.n_seq, u.h, u.bos, u.eos);
  u.nch = static_cast<int>((u.eos - u.bos + kChunk - 1) / kChunk);
  u.g0 = g0;
}
// Chunks in the lane's stream (with a plan: the planner's total, after the unit lists).
__device__ __forceinline__ int lane_total(const PrefillArgs& a, int lid) {
  if (a.lane_units) return a.lane_units[a.units + lid];
  const int nu = lane_count(a, lid);
  int t = 0;
  LaneUnit u;
  for (int i = 0; i < nu; ++i) {
    lane_unit(a, lid, i, t, u);
    t += u.nch;
  }
  return t;
}
// Consumer with the work split by token and key blocks (d_k = 128, 64 value columns):
// wave w forms the rows of token block w of E = U - W S^T and O = Qg S^T + M E, and
// owns key blocks 2w, 2w+1 of S^T (keys 32w .. 32w + 31) in fp32 accumulators.  Per
// chunk the waves exchange only the bf16 operands of the chain through LDS: wave w
// packs its keys into the S^T fragments of K step w, and its E rows into half w % 2 of
// the E fragments of K step w / 2 (permuted-K order).  Each wave loads just the
// published operands it uses (its token block of W, Qg, M, U; its key blocks of KD^T,
// e^{G_n}) straight from the ring slot into registers, one chunk ahead.  The slot of
// chunk c is released after chunk c's end-of-chunk barrier, when every wave has used
// those registers.  Over a lane's stream of units, the state of a unit is loaded
// before its first chunk and stored after its last, where the next unit's initial
// state takes the place of the updated one as the next chunk's S^T operand.
// STATES: also write the state at every chunk start (bf16, as prefill_kernel's STATES),
// and write o only when a.o is set.
template <int DK, int DV, bool STATES = false>
__device__ __forceinline__ void wy_consume_split(const PrefillArgs& a, unsigned char* smem,
                                                 __amdgpu_buffer_rsrc_t rr, int* ready,
                                                 int* done, int* abort_word, int role, int lid,
                                                 int total, int tid, int wave, int lane) {
  using SL = WySlot<DK, DV>;
  using CL = WySplitLayout;
  constexpr int KS = DK / 32, NVT = CL::NVT;
  static_assert(KS == 4, "one K step of keys per wave");
  const int lr = lane & 15, lq = lane >> 4;
  const int v0 = role * 16 * NVT;
  int* cFlag = reinterpret_cast<int*>(smem + CL::oFlag);
  const uint32_t rowO = static_cast<uint32_t>(a.H) * DV;
  auto ld16 = [&](uint32_t off) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, kDeviceScope);
  };
  auto ldf = [&](uint32_t off) -> bf16x8 { return __builtin_bit_cast(bf16x8, ld16(off)); };
  auto ldv = [&](uint32_t off) -> f32x4 { return __builtin_bit_cast(f32x4, ld16(off)); };
  const uint32_t fl = 16 * lane;
  // slot offsets of this wave's operands
  // U tiles of value blocks v0/16 + 2p, + 2p + 1 (bf16, one 16-byte piece per pair)
  auto offU = [&](int p) {
    return uint32_t(SL::oU + (wave * (SL::NVB / 2) + v0 / 32 + p) * SL::kFrag) + fl;
  };
  // W and Qg fragments are held in wave-rotated K order: register jj is K step
  // (w + jj) % 4, so jj = 0 is the wave's own key block, whose S^T operand it has in
  // registers (only the other three come from LDS)
  auto offW = [&](int jj) {
    return uint32_t(SL::oW + (wave * KS + ((wave + jj) & (KS - 1))) * SL::kFrag) + fl;
  };
  auto offQ = [&](int jj) {
    return uint32_t(SL::oQ + (wave * KS + ((wave + jj) & (KS - 1))) * SL::kFrag) + fl;
  };
  // M (w, 0) is block w; (w, 1) is block 2 + w and exists for w >= 2 (else re-read (w, 0))
  auto offM = [&](int t) {
    return uint32_t(SL::oM + (t == 0 || wave < 2 ? wave : 2 + wave) * SL::kFrag) + fl;
  };
  auto offKD = [&](int b, int t) {
    return uint32_t(SL::oKD + ((2 * wave + b) * 2 + t) * SL::kFrag) + fl;
  };
  auto offEg = [&](int b) { return uint32_t(SL::oEgn + (16 * (2 * wave + b) + 4 * lq) * 4); };
  unsigned char* sSb = smem + CL::oSb + fl;
  unsigned char* sEb = smem + CL::oEb + fl;
  unsigned char* sO = smem + CL::oO;
  auto sb_at = [&](int jj, int vt) -> bf16x8 {   // K step (w + jj) % 4
    return *reinterpret_cast<const bf16x8*>(sSb + (((wave + jj) & (KS - 1)) * NVT + vt) * 1024);
  };
  auto eb_at = [&](int t, int vt) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(sEb + (t * NVT + vt) * 1024);
  };
  // output rows of this wave (token block w) of chunk gg from its LDS tile to o for head
  // hh; rows >= `rows` of the window starting at token row cs are dropped
  auto store_rows = [&](int64_t cs, int rows, int hh, int gg) {
    const unsigned char* ob = sO + (gg & 1) * CL::kOBytes;
    // the window is the same for every lane: made wave-uniform, the buffer stores need
    // no loop over distinct descriptors
    cs = static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(
             __builtin_amdgcn_readfirstlane(static_cast<int>(cs >> 32)))) << 32) |
                              static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(cs))));
    rows = __builtin_amdgcn_readfirstlane(rows);
    hh = __builtin_amdgcn_readfirstlane(hh);
    const __amdgpu_buffer_rsrc_t win = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<bf16*>(a.o) + (cs * a.H + hh) * DV + v0, 0,
        static_cast<int>(uint32_t(rows) * rowO * 2), 0x00020000);
    // both LDS reads before either store (the compiler keeps LDS reads behind a buffer
    // store, which would serialise two read round trips)
    const int r0 = 16 * wave + lane / 8, col = 8 * (lane % 8);
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(ob + (r0 * CL::LDO + col) * 2);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(ob + ((r0 + 8) * CL::LDO + col) * 2);
    __builtin_amdgcn_raw_buffer_store_b128(x0, win, (r0 * rowO + col) * 2, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(x1, win, ((r0 + 8) * rowO + col) * 2, 0, 0);
  };

  // S^T rows of this wave: S[b][vt] holds S^T[32 w + 16 b + 4 lq + i][v0 + 16 vt + lr]
  f32x4 S[2][NVT];
  auto st_off = [&](const LaneUnit& u, int vt, int b) {
    return (static_cast<int64_t>(u.n_seq) * a.H + u.h) * DV * DK + int64_t(v0 + 16 * vt + lr) * DK +
           32 * wave + 16 * b + 4 * lq;
  };
  auto load_state = [&](const LaneUnit& u) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
        S[b][vt] = a.initial_state ? *reinterpret_cast<const f32x4*>(a.initial_state + st_off(u, vt, b))
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto store_final = [&](const LaneUnit& u) {
    if (a.final_state) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
          *reinterpret_cast<f32x4*>(a.final_state + st_off(u, vt, b)) = S[b][vt];
    }
  };
  // the lane's units: cu is the unit of the current chunk; units without chunks keep
  // their initial state.  A plan can leave a lane without units (fewer units with
  // chunks than lanes): it has nothing to do.
  const int nu = lane_count(a, lid);
  if (nu == 0) return;
  LaneUnit cu;
  int iu = 0;
  lane_unit(a, lid, 0, 0, cu);
  auto skip_empty = [&]() {
    while (cu.nch == 0) {
      if (a.final_state) {
        load_state(cu);
        store_final(cu);
      }
      if (iu + 1 >= nu) return false;
      const int g0 = cu.g0;
      lane_unit(a, lid, ++iu, g0, cu);
    }
    return true;
  };
  if (skip_empty()) load_state(cu);
  // this wave's K step of the S^T operand, packed once per chunk: written to LDS for
  // the other waves and kept in registers for its own products of the next chunk
  bf16x8 sown[NVT];
#pragma unroll
  for (int vt = 0; vt < NVT; ++vt) {
    sown[vt] = pack_frag(S[0][vt], S[1][vt]);
    *reinterpret_cast<bf16x8*>(sSb + (wave * NVT + vt) * 1024) = sown[vt];
  }

  // this chunk's operands; each is reloaded from the next chunk's slot right after its
  // last use here, so a request has about one chunk of time to arrive
  bf16x8 U[NVT / 2];
  f32x4 Uw[NVT];   // U widened to fp32: the E accumulators' initial values
  f32x4 eg[2];
  bf16x8 Wf[KS], Qf[KS], Mf[2], KDf[2][2];
  auto load_w = [&](uint32_t slot) {
#pragma unroll
    for (int j = 0; j < KS; ++j) Wf[j] = ldf(slot + offW(j));
  };
  auto load_q = [&](uint32_t slot) {
#pragma unroll
    for (int j = 0; j < KS; ++j) Qf[j] = ldf(slot + offQ(j));
  };
  auto load_m = [&](uint32_t slot) {
#pragma unroll
    for (int t = 0; t < 2; ++t) Mf[t] = ldf(slot + offM(t));
  };
  auto load_kd = [&](uint32_t slot) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 2; ++t) KDf[b][t] = ldf(slot + offKD(b, t));
  };
  auto load_eg = [&](uint32_t slot) {
#pragma unroll
    for (int b = 0; b < 2; ++b) eg[b] = ldv(slot + offEg(b));
  };

  bool ok = true, nok = true;
  if (total > 0) {
    if (tid == 0) cFlag[0] = wait_at_least(ready, 1, abort_word) ? 1 : 0;
    lds_barrier();
    ok = cFlag[0] != 0;
    if (ok) {
#pragma unroll
      for (int p = 0; p < NVT / 2; ++p) U[p] = ldf(offU(p));
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt)
        Uw[vt] = vt % 2 ? widen(bf16x4{U[vt / 2][4], U[vt / 2][5], U[vt / 2][6], U[vt / 2][7]})
                        : widen(bf16x4{U[vt / 2][0], U[vt / 2][1], U[vt / 2][2], U[vt / 2][3]});
      // the order of the loop's own requests (U, W, e^{G_n}, Qg, M, KD^T), so the
      // compiler's count of loads in flight agrees on both paths into the loop
      load_w(0);
      load_eg(0);
      load_q(0);
      load_m(0);
      load_kd(0);
    }
    if (tid == 0) cFlag[1] = total > 1 ? (wait_at_least(ready + 1 % a.R, 2, abort_word) ? 1 : 0) : 1;
    lds_barrier();
    nok = cFlag[1] != 0;
  }

  // ring slot indices of chunks g - 1, g, g + 1, g + 2
  int sp = 0, s0 = 0, s1 = 1 % a.R, s2 = 2 % a.R;
  const int t_own = wave >> 1, h_own = wave & 1;
  const bool write_o = !STATES || a.o != nullptr;
  // the producers' Qg leaves the query scale out in the forward kernel (kept for the
  // backward's chain tiles): it is applied to each output tile here
  const float oscale = STATES ? 1.f : a.scale;
  f32x4 Ot[NVT];
  // the o window of the previous chunk (its rows leave during this chunk)
  int64_t pc0 = 0;
  int prows = 0, ph = 0, punit = -1;
  int g = 0;
  KDA_PHASE(PhaseClock phc; phc.start();)
  // Outer loop: the lane's units with chunks; inner loop: the chunks of one unit.  The
  // unit's bounds are fixed over the inner loop, and everything that moves to the next
  // unit lives outside it, so the per-chunk path carries no lane bookkeeping.
  while (ok && g < total) {
    const int uend = cu.g0 + cu.nch;                             // stream index past the unit
    const int64_t cbase = cu.bos - int64_t(cu.g0) * kChunk;      // chunk g starts at cbase + 64 g
    const int64_t ueos = cu.eos;
    const int uh = cu.h;
    [[maybe_unused]] const int64_t sbase =                       // chunk g's state slot (STATES)
        STATES ? chunk_slot_base(cu.n_seq, cu.bos) - cu.g0 : 0;
    // STATES: the state at the start of chunk g as bf16 into its slot (non-temporal, as
    // every checkpoint and tile store: read only by later kernels).  Issued after the
    // chunk's operand requests: loads complete in issue order, so a store issued before
    // them would make the next chunk wait for its write to memory as well.  With `keep`
    // false the buffer range is empty and the stores are dropped, so every chunk issues
    // the same instructions.
    [[maybe_unused]] auto store_ckpt = [&](int gg, bool keep) {
      const __amdgpu_buffer_rsrc_t ck = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<bf16*>(a.chunk_states) + ((sbase + (keep ? gg : cu.g0)) * a.H + uh) * DV * DK, 0,
          keep ? DV * DK * 2 : 0, 0x00020000);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          const f32x4 x = S[b][vt];
          const bf16x4 y = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]),
                                  static_cast<bf16>(x[2]), static_cast<bf16>(x[3])};
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(u32x2, y), ck,
              ((v0 + 16 * vt + lr) * DK + 32 * wave + 16 * b + 4 * lq) * 2, 0, kNonTemporal);
        }
    };
    if constexpr (STATES) store_ckpt(cu.g0, true);   // the unit's initial state
    for (; ok && g < uend; ++g) {
      KDA_PHASE(phc.mark(0);)
      const int64_t c0 = cbase + int64_t(g) * kChunk;
      const bool has_next = g + 1 < total, has2 = g + 2 < total;
      int fv = 0;
      if (tid == 0 && has2)
        fv = __hip_atomic_load(ready + s2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The next chunk's operands are requested unconditionally (past the last chunk
      // they are unused bytes of an idle slot).
      const uint32_t nslot = static_cast<uint32_t>(s1) * SL::kBytes;

      f32x4 E[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        E[vt] = Uw[vt];
        Ot[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int p = 0; p < NVT / 2; ++p) U[p] = ldf(nslot + offU(p));
      // E = U - W S^T for token block w; the S^T fragments stay for O.  The wave's own K
      // step is its state packed as written to LDS at the end of the last chunk.
      bf16x8 sb[KS][NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) sb[0][vt] = sown[vt];
#pragma unroll
      for (int j = 1; j < KS; ++j)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) sb[j][vt] = sb_at(j, vt);
#pragma unroll
      for (int j = 0; j < KS; ++j)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) E[vt] = mma_bf16(Wf[j], sb[j][vt], E[vt]);
      KDA_PHASE(phc.mark(1);)
      load_w(nslot);
      // this wave's E rows into its half of the E operand fragments
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const f32x4 e = E[vt];
        *reinterpret_cast<bf16x4*>(sEb + (t_own * NVT + vt) * 1024 + 8 * h_own) =
            bf16x4{static_cast<bf16>(e[0]), static_cast<bf16>(e[1]), static_cast<bf16>(e[2]),
                   static_cast<bf16>(e[3])};
      }
      // D S^T for this wave's keys, while the E products run: the empty asm keeps the
      // multiplies ahead of the barrier (the compiler would otherwise sink them to the
      // state update, where they delay its products)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          S[b][vt] *= eg[b];
          asm volatile("" : "+v"(S[b][vt]));
        }
      // the next chunk's e^{G_n}, right after its last use: requested here rather than
      // with KD^T at the chunk's end, its wait in the next chunk's E phase does not
      // also wait for the operand requests that follow it
      load_eg(nslot);
      lds_barrier();
      KDA_PHASE(phc.mark(2);)
      bf16x8 eb[2][NVT];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) eb[t][vt] = eb_at(t, vt);
      // O = Qg S^T + M E (token block w reads E blocks <= w: K step 1 only for w >= 2)
#pragma unroll
      for (int j = 0; j < KS; ++j)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) Ot[vt] = mma_bf16(sb[j][vt], Qf[j], Ot[vt]);
      load_q(nslot);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) Ot[vt] = mma_bf16(eb[0][vt], Mf[0], Ot[vt]);
      if (wave >= 2) {
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) Ot[vt] = mma_bf16(eb[1][vt], Mf[1], Ot[vt]);
      }
      load_m(nslot);
      KDA_PHASE(phc.mark(3);)
      // S^T += KD^T E for this wave's keys
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) S[b][vt] = mma_bf16(KDf[b][t], eb[t][vt], S[b][vt]);
      KDA_PHASE(phc.mark(4);)
      // this chunk's output rows into its LDS tile while the state products run (the
      // other tile holds the previous chunk's rows until they are stored below)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const f32x4 x = Ot[vt] * oscale;
        *reinterpret_cast<bf16x4*>(sO + (g & 1) * CL::kOBytes +
                                   ((16 * wave + lr) * CL::LDO + 16 * vt + 4 * lq) * 2) =
            bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                   static_cast<bf16>(x[3])};
      }
      // the next chunk's U (requested at this chunk's start) widened while the state
      // products run
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        Uw[vt] = vt % 2 ? widen(bf16x4{U[vt / 2][4], U[vt / 2][5], U[vt / 2][6], U[vt / 2][7]})
                        : widen(bf16x4{U[vt / 2][0], U[vt / 2][1], U[vt / 2][2], U[vt / 2][3]});
        asm volatile("" : "+v"(Uw[vt]));   // here, not after the end-of-chunk barrier
      }
      load_kd(nslot);
      // the previous chunk's output rows, from this wave's LDS rows (after the operand
      // requests: stores complete in order with the loads, and the next chunk waits
      // for those)
      if (g > 0 && write_o) store_rows(pc0, prows, ph, g - 1);
      // every wave has used chunk g - 1's operands (at the last barrier): its slot is
      // free.  Released here, after the operand requests, for the same reason.
      if (tid == 0 && g > 0) __hip_atomic_fetch_add(done + sp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // this chunk's o window
      pc0 = c0;
      prows = static_cast<int>(min(ueos - c0, static_cast<int64_t>(kChunk)));
      ph = uh;
      // the next chunk's S^T operand (K step w)
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        sown[vt] = pack_frag(S[0][vt], S[1][vt]);
        *reinterpret_cast<bf16x8*>(sSb + (wave * NVT + vt) * 1024) = sown[vt];
      }
      // S^T is now the state at the start of chunk g + 1 (none after the unit's last)
      if constexpr (STATES) store_ckpt(g + 1, g + 1 < uend);

      if (tid == 0)
        cFlag[g & 1] = !has2 ? 1
                             : ((fv >= g + 3 || wait_at_least(ready + s2, g + 3, abort_word)) ? 1 : 0);
      KDA_PHASE(phc.mark(5);)
      lds_barrier();
      KDA_PHASE(phc.mark(6); phc.close(7);)
      ok = has_next ? nok : true;
      nok = cFlag[g & 1] != 0;
      sp = s0;
      s0 = s1;
      s1 = s2;
      s2 = s2 + 1 == a.R ? 0 : s2 + 1;
    }
    punit = cu.unit;
    if (g < uend) break;   // a hand-off aborted inside the unit
    // the unit is complete: its final state; then the next unit with chunks, whose
    // initial state replaces this wave's S^T operand fragments (the end-of-chunk
    // barrier above has ordered every read of the old ones)
    store_final(cu);
    if (g >= total) break;
    lane_unit(a, lid, ++iu, uend, cu);
    skip_empty();
    load_state(cu);
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      sown[vt] = pack_frag(S[0][vt], S[1][vt]);
      *reinterpret_cast<bf16x8*>(sSb + (wave * NVT + vt) * 1024) = sown[vt];
    }
    lds_barrier();
  }

  KDA_PHASE(phc.write(tid, role);)
  // the last chunk's output rows (written before the loop's last barrier)
  if (ok && total > 0 && write_o) store_rows(pc0, prows, ph, g - 1);
  // units after the last one with chunks: empty, they keep their initial state
  if (ok && total > 0) {
    while (iu + 1 < nu) {
      const int g0 = cu.g0 + cu.nch;
      lane_unit(a, lid, ++iu, g0, cu);
      if (a.final_state) {
        load_state(cu);
        store_final(cu);
      }
    }
  }
  if (!ok) {
    // the rows of the last completed chunk are valid; when they belong to an earlier
    // unit than the one in progress they are stored (otherwise that unit is poisoned)
    if (punit >= 0 && punit != cu.unit && write_o) store_rows(pc0, prows, ph, g - 1);
    // the unit in progress and every later one did not complete
    for (;;) {
      poison_outputs<DK, DV, STATES>(a, cu.n_seq, cu.h, cu.bos, cu.eos, cu.nch, v0, 16 * NVT, tid);
      if (iu + 1 >= nu) break;
      const int g0 = cu.g0 + cu.nch;
      lane_unit(a, lid, ++iu, g0, cu);
    }
  }
}

// A producer's chunk tiles for the backward's reverse chain (ChainTiles): KD, Qg^T, -W^T
// fragments and e^{G_n} from its LDS; of M, products<true>() wrote the blocks on and
// below the diagonal, the blocks above it are zero.
template <int DK, int DV>
__device__ __forceinline__ void publish_chain_tiles(const unsigned char* smem, unsigned char* dst,
                                                    int tid, int wave, int lane) {
  using TL = ChainTiles<DK>;
  using PL = WyProducerLayout<DK, DV>;
  // KD, Qg^T, -W^T (staged in the A area by publish_wu) and e^{G_n} from LDS; the
  // lower blocks of M were written from their accumulators, its upper blocks are zero
  store_kd_frags<DK>(dst, reinterpret_cast<const bf16*>(smem + PL::oKD), PL::LDK, nullptr, false,
                     wave, lane);
  store_tr_frags<DK>(dst + TL::oQT, reinterpret_cast<const bf16*>(smem + PL::oQg), PL::LDK, wave,
                     lane);
  store_tr_frags<DK>(dst + TL::oWT, reinterpret_cast<const bf16*>(smem + PL::oA), PL::LDK, wave,
                     lane);
  for (int q = tid; q < TL::PC; q += kThreads)
    if ((8 * (q % 8)) / 16 > (q / 8) / 16)
      __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u},
                                  reinterpret_cast<u32x4*>(dst + TL::oM + 16 * size_t(q)));
  store_egn<DK>(dst, reinterpret_cast<const float*>(smem + PL::oEgn), tid);
}

template <int DK, int DV>
struct WyLds {
  static constexpr size_t kCons = WyConsumerLayout<DK, DV>::kBytes > WySplitLayout::kBytes
                                      ? WyConsumerLayout<DK, DV>::kBytes
                                      : WySplitLayout::kBytes;
  static constexpr size_t kProd = WyProducerLayout<DK, DV>::kBytes;
  static constexpr size_t kBytes = kProd > kCons ? kProd : kCons;
  static_assert(kBytes <= 160 * 1024, "LDS budget exceeded");
};

// Per unit: NC consumers of 4 * VBW value columns (wave w of consumer r owns columns
// 4 VBW r + VBW w .. +VBW) and NP producers (producer p takes chunks p, p + NP, ...).
// DECAY as for prefill_kernel.
// STATES: see wy_consume_split (d_k = 128 with 16-column waves only).
template <int DK, int DV, int VBW, int DECAY, bool STATES = false>
__global__ __launch_bounds__(kThreads, 1) void prefill_wy_kernel(PrefillArgs a) {
  static_assert(!STATES || (DK == 128 && VBW == 16), "chunk states from the split consumer only");
  using PR = WyProducer<DK, DV>;
  using SL = WySlot<DK, DV>;
  using PL = WyProducerLayout<DK, DV>;
  constexpr int KS = DK / 32, NKB = DK / 16, NVS = VBW / 16;

  __shared__ __attribute__((aligned(16))) unsigned char smem[WyLds<DK, DV>::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  const int W = a.NC + a.NP;
  int lid, role;
  unit_role(blockIdx.x, W, a.lanes, a.xcd_remap, lid, role);
  const int total = lane_total(a, lid);

  int* abort_word = reinterpret_cast<int*>(a.workspace);
  int* ready = reinterpret_cast<int*>(a.workspace + kWsHeader + coop_plan_bytes(a)) +
               size_t(lid) * coop_flag_words(a.R);
  int* done = ready + a.R;
  int* arrive = done + a.R;
  unsigned char* ring = a.workspace + kWsHeader + coop_plan_bytes(a) +
                        coop_flags_bytes(a.lanes, a.R) + size_t(lid) * a.R * SL::kBytes;
  const __amdgpu_buffer_rsrc_t rr = ring_rsrc(ring, static_cast<uint32_t>(a.R * SL::kBytes));

  // Co-location.  When every workgroup of the unit runs on the XCD its id was dealt
  // to (ids congruent mod 8, read back from XCC_ID), they share one L2: producers then
  // publish with plain stores, which the consumers' device-scope loads read from that
  // L2.  Otherwise producers store device-scope (written through past the L2).  Each
  // workgroup adds 1 (on its XCD) or 1 << 16 (elsewhere) to the unit's arrive word.
  if (tid == 0) {
    const int xcc = static_cast<int>(__builtin_amdgcn_s_getreg(kHwRegXccId) & 0xf);
    const bool here = a.xcd_remap != 0 && xcc == static_cast<int>(blockIdx.x & 7);
    __hip_atomic_fetch_add(arrive, here ? 1 : 0x10000, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (role >= a.NC) {
    // ================================ producer ==================================
    const int p = role - a.NC;
    PR pr;
    pr.init(smem, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k),
            static_cast<const bf16*>(a.v), a.g, a.beta, a.H, 0, a.scale, tid, wave, a.flags);
    int* pFlag = reinterpret_cast<int*>(smem + PL::oFlag);
    if (tid == 0) {
      int mode = -1;
      for (uint32_t it = 0; it < kSpinLimit; ++it) {
        const int v = __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((v & 0xffff) + (v >> 16) >= W) {
          mode = (v >> 16) == 0 ? 1 : 0;
          break;
        }
        if ((it & 15) == 15 &&
            __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
          break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (mode < 0) raise_abort(abort_word);
      pFlag[1] = mode;
    }
    lds_barrier();
    if (pFlag[1] < 0 || total == 0) return;
    pr.local = pFlag[1] == 1;
    // Producer p takes chunks p, p + NP, ... of the lane's stream.  During chunk g it
    // loads the inputs of chunk g + NP, whose unit is followed by one cursor (index in
    // the lane, stream end, row base, end row, head); that unit is the next iteration's
    // own, so per chunk only the stream end is compared.
    if (p >= total) return;
    int ix = 0;
    LaneUnit ux;
    lane_unit(a, lid, 0, 0, ux);
    int xend = ux.g0 + ux.nch, xh = ux.h;
    int64_t xbase = ux.bos - int64_t(ux.g0) * kChunk, xeos = ux.eos;
    [[maybe_unused]] int64_t xslot = STATES ? chunk_slot_base(ux.n_seq, ux.bos) - ux.g0 : 0;
    auto seek = [&](int gg) {
      while (__builtin_expect(gg >= xend, 0)) {
        lane_unit(a, lid, ++ix, xend, ux);
        xend = ux.g0 + ux.nch;
        xh = ux.h;
        xbase = ux.bos - int64_t(ux.g0) * kChunk;
        xeos = ux.eos;
        if constexpr (STATES) xslot = chunk_slot_base(ux.n_seq, ux.bos) - ux.g0;
      }
    };
    seek(p);
    // chunk g: first row, rows, head and (STATES) chunk slot
    int64_t c0 = xbase + int64_t(p) * kChunk;
    int n = static_cast<int>(min(xeos - c0, static_cast<int64_t>(kChunk)));
    [[maybe_unused]] int ch = xh;
    [[maybe_unused]] int64_t cslot = xslot + p;
    pr.template load<DECAY, !STATES>(c0, n, xh);
    // ring slot of chunk g and the releases it needs: g mod R, NC * (g div R)
    int s = p % a.R, need = a.NC * (p / a.R);
    KDA_PHASE(PhaseClock phc; phc.start();)
    for (int g = p; g < total; g += a.NP) {
      KDA_PHASE(phc.mark(0);)
      const int gn = g + a.NP;
      const bool has_next = gn < total;
      if (has_next) seek(gn);
      const int64_t c1 = xbase + int64_t(gn) * kChunk;
      const int n1 = static_cast<int>(min(xeos - c1, static_cast<int64_t>(kChunk)));
      // the slot must have been released by every consumer of its previous chunk; its
      // counter is read before the factors, so the check after them rarely waits
      int dv = 0;
      if (tid == 0) dv = __hip_atomic_load(done + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pr.template factors<DECAY, STATES>(n, g + 1);
      KDA_PHASE(phc.mark(1);)
      if (tid == 0) pFlag[0] = (dv >= need || wait_at_least(done + s, need, abort_word)) ? 1 : 0;
      lds_barrier();
      if (pFlag[0] == 0) break;
      KDA_PHASE(phc.mark(2);)
      const uint32_t slot = static_cast<uint32_t>(s) * SL::kBytes;
      // STATES: this chunk's tiles for the backward's reverse chain
      [[maybe_unused]] unsigned char* tiles = nullptr;
      if constexpr (STATES)
        tiles = static_cast<unsigned char*>(a.chunk_tiles) + (cslot * a.H + ch) * ChainTiles<DK>::kBytes;
      // the next chunk's inputs are requested in slices between the phases, none of
      // them in the phase that publishes W and U.  Without a next chunk the slices
      // re-read this chunk's rows (unused): the loads stay unconditional, so the code
      // has no branches around them and the compiler can count them exactly.
      constexpr int L = PR::kLoads, RPG = PR::RPG;
      const int64_t cl = has_next ? c1 : c0;
      const int nl = has_next ? n1 : n;
      const int hl = xh;   // chunk g + NP's head, or chunk g's when there is none
      pr.template load_slice<DECAY, 0, RPG / 2, !STATES>(cl, nl, hl);            // g, first half
      pr.template load_slice<DECAY, PR::kSB, L, !STATES>(cl, nl, hl);            // beta
      if constexpr (STATES)
        pr.template products<true>(rr, slot, reinterpret_cast<bf16*>(tiles + ChainTiles<DK>::oM));
      else
        pr.products(rr, slot);
      pr.template load_slice<DECAY, RPG / 2, RPG, !STATES>(cl, nl, hl);          // g, second half
      lds_barrier();
      KDA_PHASE(phc.mark(3);)
      pr.template load_slice<DECAY, PR::kSK, PR::kSQ, !STATES>(cl, nl, hl);      // k
      pr.template load_slice<DECAY, PR::kSV, PR::kSB, !STATES>(cl, nl, hl);      // v
      pr.inverse_blocks();
      lds_barrier();
      KDA_PHASE(phc.mark(4);)
      // waves 0, 1 merge the diagonal pairs; the Qg / KD^T fragments are spread over
      // all four waves
      if (wave < 2) pr.inverse_pairs();
      pr.template publish_qk<0, 4>(rr, slot);
      pr.template load_slice<DECAY, PR::kSQ, PR::kSV, !STATES>(cl, nl, hl);      // q
      lds_barrier();
      KDA_PHASE(phc.mark(5);)
      pr.inverse_rest();
      KDA_PHASE(phc.mark(6);)
      if constexpr (STATES) {
        // -W rows staged in the A area (dead after the inverse) for the transposed copy
        static_assert(size_t(kChunk) * PL::LDK * 2 <= PL::oX - PL::oA, "-W staging fits");
        pr.template publish_wu<true>(rr, slot, reinterpret_cast<bf16*>(smem + PL::oA));
        pr.qg_to_chunk_start();
        lds_barrier();
        publish_chain_tiles<DK, DV>(smem, tiles, tid, wave, lane);
      } else {
        pr.publish_wu(rr, slot);
      }
      KDA_PHASE(phc.mark(7);)
      // every slot store of the workgroup acknowledged (device-visible), then publish
      vm_barrier();
      if (tid == 0) __hip_atomic_store(ready + s, g + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      KDA_PHASE(phc.mark(8); phc.close(9);)
      c0 = c1;
      n = n1;
      ch = xh;
      cslot = xslot + gn;
      s += a.NP;
      while (s >= a.R) {
        s -= a.R;
        need += a.NC;
      }
    }
    KDA_PHASE(phc.write(tid, 100 + p);)
    return;
  }

  // ================================== consumer =====================================
  if constexpr (DK == 128 && VBW == 16) {
    wy_consume_split<DK, DV, STATES>(a, smem, rr, ready, done, abort_word, role, lid, total, tid,
                                     wave, lane);
    return;
  }
  // the value-column consumer serves one unit per lane (no lane plan)
  LaneUnit u0;
  lane_unit(a, lid, 0, 0, u0);
  const int n_seq = u0.n_seq, h = u0.h, nch = u0.nch;
  const int64_t bos = u0.bos, eos = u0.eos;
  const int vw0 = role * 4 * VBW + VBW * wave;     // this wave's first value column
  using CL = WyConsumerLayout<DK, DV>;
  int* cFlag = reinterpret_cast<int*>(smem + CL::oFlag);
  const uint32_t rowO = static_cast<uint32_t>(a.H) * DV;
  constexpr int BV = 4 * VBW;
  const int v0 = role * BV;
  // Output tiles go through LDS and leave as whole 2*BV-byte rows during the next
  // chunk: wave w stores rows 16 w .. 16 w + 15, LPR lanes per row, NOI stores.
  constexpr int LPR = BV / 8, RPI = 64 / LPR, NOI = 16 / RPI;
  auto o_window = [&](int64_t cs, int rows) {   // rows >= `rows` fall outside
    return __builtin_amdgcn_make_buffer_rsrc(static_cast<bf16*>(a.o) + (cs * a.H + h) * DV + v0, 0,
                                             static_cast<int>(uint32_t(rows) * rowO * 2), 0x00020000);
  };
  auto o_read = [&](const unsigned char* ob, int i) -> u32x4 {
    const int r = 16 * wave + RPI * i + lane / LPR, col = 8 * (lane % LPR);
    return *reinterpret_cast<const u32x4*>(ob + (r * CL::LDO + col) * 2);
  };
  auto o_store = [&](__amdgpu_buffer_rsrc_t w, int i, u32x4 x) {
    const int r = 16 * wave + RPI * i + lane / LPR, col = 8 * (lane % LPR);
    __builtin_amdgcn_raw_buffer_store_b128(x, w, (r * rowO + col) * 2, 0, 0);
  };

  // S^T tiles: S[kb][vs] holds S^T[16 kb + 4 lq + i][vw0 + 16 vs + lr]
  f32x4 S[NKB][NVS];
  bf16x8 Sb[KS][NVS];
  const int64_t st_base = (static_cast<int64_t>(n_seq) * a.H + h) * DV * DK;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
      S[kb][vs] = a.initial_state
                      ? *reinterpret_cast<const f32x4*>(a.initial_state + st_base +
                                                        int64_t(vw0 + 16 * vs + lr) * DK +
                                                        16 * kb + 4 * lq)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) Sb[j][vs] = pack_frag(S[2 * j][vs], S[2 * j + 1][vs]);

  f32x4 U[4][NVS];
  constexpr int kShare = SL::nStage / 4;   // staged blocks copied by each wave
  auto stage_blk = [&](uint32_t slot, unsigned char* buf, int i) {
    const int blk = wave + 4 * i;
    ring_to_lds(rr, slot + blk * SL::kFrag, buf + blk * SL::kFrag, lane);
  };
  auto load_u = [&](uint32_t slot, int k) {   // k = tb * NVS + vs
    const int tb = k / NVS, vs = k % NVS;
    const int vb = vw0 / 16 + vs;
    const bf16x8 u = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
        rr, slot + SL::oU + (tb * (SL::NVB / 2) + vb / 2) * SL::kFrag + 16 * lane, 0,
        kDeviceScope));
    U[tb][vs] = vb % 2 ? widen(bf16x4{u[4], u[5], u[6], u[7]}) : widen(bf16x4{u[0], u[1], u[2], u[3]});
  };

  bool ok = true, nok = true;
  if (nch > 0) {
    if (tid == 0) cFlag[0] = wait_at_least(ready, 1, abort_word) ? 1 : 0;
    lds_barrier();
    ok = cFlag[0] != 0;
    if (ok) {
#pragma unroll
      for (int i = 0; i < kShare; ++i) stage_blk(0, smem, i);
#pragma unroll
      for (int k = 0; k < 4 * NVS; ++k) load_u(0, k);
    }
    if (tid == 0) cFlag[1] = nch > 1 ? (wait_at_least(ready + 1 % a.R, 2, abort_word) ? 1 : 0) : 1;
    vm_barrier();
    nok = cFlag[1] != 0;
  }

  // One chunk is a fixed stream of LDS reads, each feeding NVS MFMAs (or a row scale),
  // read P steps ahead of use:
  //   W (j, tb)       E[tb]  += W S^T
  //   Q (j, tb), egn  Ot[tb] += S Qg^T; every third step instead reads e^{G_n} for one
  //                   key block and scales those rows of S^T (D S^T), in the shadow of
  //                   the neighbouring MFMAs; E is packed to bf16 early in this phase
  //   M (tb, t)       Ot[tb] += E^T M^T
  //   KD (t, kb)      S^T[kb] += KD^T E; the next chunk's bf16 S^T operand is packed
  //                   during the second pass
  // The next chunk's U tiles and staged blocks are requested at evenly spaced steps,
  // so the vector-memory traffic overlaps the MFMA and LDS work.
  constexpr int NW = 4 * KS, NM = 6;
  constexpr int iQ = NW, iM = iQ + 3 * NKB, iKD = iM + NM, NF = iKD + 2 * NKB;
  static_assert(NW == 2 * NKB, "Q and egn entries interleave two to one");
  constexpr int P = 6;
  // U load k at step kU0 + 3 k; staged block i at step kD0 + kDs i
  constexpr int kU0 = 1, kD0 = 2, kDs = (NF - kD0 - 2) / kShare;
  static_assert(kDs >= 1 && kD0 + kDs * (kShare - 1) < NF && kU0 + 3 * (4 * NVS - 1) < NF,
                "memory requests do not fit the stream");
  auto frag_at = [&](const unsigned char* F, int i) -> u32x4 {
    uint32_t off;
    if (i < iQ) {
      off = SL::oW + ((i % 4) * KS + i / 4) * SL::kFrag + 16 * lane;
    } else if (i < iM) {
      const int r = i - iQ;
      if (r % 3 == 2) {
        off = SL::oEgn + (16 * (r / 3) + 4 * lq) * 4;
      } else {
        const int k = 2 * (r / 3) + r % 3;
        off = SL::oQ + ((k % 4) * KS + k / 4) * SL::kFrag + 16 * lane;
      }
    } else if (i < iKD) {
      // blocks (tb, 0) for tb < 4, then (2, 1), (3, 1): stored in this order
      off = SL::oM + (i - iM) * SL::kFrag + 16 * lane;
    } else {
      const int k = i - iKD, t = k / NKB, kb = k % NKB;
      off = SL::oKD + (kb * 2 + t) * SL::kFrag + 16 * lane;
    }
    return *reinterpret_cast<const u32x4*>(F + off);
  };

  // ring slot indices of chunks c, c + 1, c + 2
  int s0 = 0, s1 = 1 % a.R, s2 = 2 % a.R;
  for (int c = 0; ok && c < nch; ++c) {
    const int64_t c0 = bos + int64_t(c) * kChunk;
    const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
    const bool has_next = c + 1 < nch, has2 = c + 2 < nch;
    const unsigned char* F = smem + (c & 1) * SL::kStage;
    // chunk c is in LDS and U: its slot is free
    if (tid == 0) __hip_atomic_fetch_add(done + s0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the flag of chunk c + 2, checked at the end of this chunk
    int fv = 0;
    if (tid == 0 && has2)
      fv = __hip_atomic_load(ready + s2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The next chunk is requested unconditionally (a slot that is not ready yet, or
    // past the last chunk, only fills the idle buffer with unused bytes).
    const uint32_t nslot = static_cast<uint32_t>(s1) * SL::kBytes;
    unsigned char* nbuf = smem + ((c + 1) & 1) * SL::kStage;
    // this chunk's output tile, and the previous chunk's (stored during this stream;
    // an empty window for c = 0 drops those stores)
    unsigned char* Ocur = smem + CL::oO + (c & 1) * CL::kOBytes;
    const unsigned char* Oprev = smem + CL::oO + ((c + 1) & 1) * CL::kOBytes;
    const __amdgpu_buffer_rsrc_t owin = o_window(c0 - kChunk, c > 0 ? kChunk : 0);
    u32x4 ox[NOI];

    f32x4 E[4][NVS], Ot[4][NVS];
    bf16x8 Eb[2][NVS];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        E[tb][vs] = U[tb][vs];
        Ot[tb][vs] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    u32x4 fb[P + 1];
    static_for<P>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      fb[i] = frag_at(F, i);
    });
    __builtin_amdgcn_sched_barrier(0);
    static_for<NF>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + P < NF) fb[(i + P) % (P + 1)] = frag_at(F, i + P);
      if constexpr (i >= kU0 && (i - kU0) % 3 == 0 && (i - kU0) / 3 < 4 * NVS)
        load_u(nslot, (i - kU0) / 3);
      if constexpr (i >= kD0 && (i - kD0) % kDs == 0 && (i - kD0) / kDs < kShare)
        stage_blk(nslot, nbuf, (i - kD0) / kDs);
      // the previous chunk's outputs: LDS reads at steps iQ + 2m, stores two steps later
      if constexpr (i >= iQ && i < iQ + 2 * NOI && (i - iQ) % 2 == 0)
        ox[(i - iQ) / 2] = o_read(Oprev, (i - iQ) / 2);
      if constexpr (i >= iQ + 2 && i < iQ + 2 + 2 * NOI && (i - iQ) % 2 == 0)
        o_store(owin, (i - iQ - 2) / 2, ox[(i - iQ - 2) / 2]);
      const u32x4 raw = fb[i % (P + 1)];
      const bf16x8 f = __builtin_bit_cast(bf16x8, raw);
      if constexpr (i < iQ) {
        constexpr int j = i / 4, tb = i % 4;
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs) E[tb][vs] = mma_bf16(f, Sb[j][vs], E[tb][vs]);
      } else if constexpr (i < iM) {
        constexpr int r = i - iQ;
        if constexpr (r % 3 == 2) {
          // rows 16 kb + 4 lq + i of S^T scaled by e^{G_n}
          constexpr int kb = r / 3;
          const f32x4 dd = __builtin_bit_cast(f32x4, raw);
#pragma unroll
          for (int vs = 0; vs < NVS; ++vs) S[kb][vs] *= dd;
        } else {
          constexpr int k = 2 * (r / 3) + r % 3, j = k / 4, tb = k % 4;
#pragma unroll
          for (int vs = 0; vs < NVS; ++vs) Ot[tb][vs] = mma_bf16(Sb[j][vs], f, Ot[tb][vs]);
        }
        // E is final since the last W step: pack it while the Qg products run
        if constexpr (r == 3 || r == 7) {
          constexpr int t = r == 3 ? 0 : 1;
#pragma unroll
          for (int vs = 0; vs < NVS; ++vs) Eb[t][vs] = pack_frag(E[2 * t][vs], E[2 * t + 1][vs]);
        }
      } else if constexpr (i < iKD) {
        constexpr int k = i - iM, tb = k < 4 ? k : k - 2, t = k < 4 ? 0 : 1;
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs) Ot[tb][vs] = mma_bf16(Eb[t][vs], f, Ot[tb][vs]);
      } else {
        constexpr int k = i - iKD, t = k / NKB, kb = k % NKB;
        if constexpr (k < 4 * NVS) {
          // output tile (tb, vs) into LDS: 4 consecutive value columns of token 16 tb + lr
          constexpr int tb = k / NVS, vs = k % NVS;
          const f32x4 x = Ot[tb][vs] * a.scale;
          *reinterpret_cast<bf16x4*>(Ocur + ((16 * tb + lr) * CL::LDO + VBW * wave + 16 * vs + 4 * lq) * 2) =
              bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                     static_cast<bf16>(x[3])};
        }
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs) S[kb][vs] = mma_bf16(f, Eb[t][vs], S[kb][vs]);
        // second pass: key blocks 2j, 2j+1 are final two steps after 2j+1 was issued
        if constexpr (t == 1 && kb >= 3 && kb % 2 == 1) {
          constexpr int j = (kb - 3) / 2;
#pragma unroll
          for (int vs = 0; vs < NVS; ++vs) Sb[j][vs] = pack_frag(S[2 * j][vs], S[2 * j + 1][vs]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // the key-block pairs not packed inside the stream
#pragma unroll
    for (int j = (NKB - 2) / 2; j < KS; ++j)
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) Sb[j][vs] = pack_frag(S[2 * j][vs], S[2 * j + 1][vs]);

    if (tid == 0)
      cFlag[c & 1] = !has2 ? 1
                           : ((fv >= c + 3 || wait_at_least(ready + s2, c + 3, abort_word)) ? 1 : 0);
    vm_barrier();
    ok = has_next ? nok : true;
    nok = cFlag[c & 1] != 0;
    s0 = s1;
    s1 = s2;
    s2 = s2 + 1 == a.R ? 0 : s2 + 1;
  }

  // the last chunk's outputs (its tile was completed before the loop's last barrier)
  if (ok && nch > 0) {
    const int64_t cl = bos + int64_t(nch - 1) * kChunk;
    const __amdgpu_buffer_rsrc_t owin = o_window(cl, static_cast<int>(eos - cl));
    const unsigned char* Olast = smem + CL::oO + ((nch - 1) & 1) * CL::kOBytes;
#pragma unroll
    for (int i = 0; i < NOI; ++i) o_store(owin, i, o_read(Olast, i));
  }

  if (ok && a.final_state) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs)
        *reinterpret_cast<f32x4*>(a.final_state + st_base + int64_t(vw0 + 16 * vs + lr) * DK +
                                  16 * kb + 4 * lq) = S[kb][vs];
  }
  if (!ok) poison_outputs<DK, DV, false>(a, n_seq, h, bos, eos, nch, v0, BV, tid);
}

// Before a producer/consumer launch (one wave): zero the abort word and the hand-off
// flags (not the sticky abort word 1).  With a lane plan, spread the units over the
// lanes: sequences longest first (ties: lower index), each of a sequence's H units to
// the lane with the fewest chunks so far (ties: the lower lane), so that the lanes'
// chunk streams come out nearly equal and the longest units start first.
constexpr int kPlanMaxSeqs = 256, kPlanMaxUnits = 8192, kPlanMaxLanes = 64;

// Minimum of v over the 64 lanes of the wave, returned to every lane: DPP steps within
// each row of 16 lanes (shift right by 1, 2, 4, 8), then the row minima joined by the
// row broadcasts of lanes 15 and 31; lane 63 ends with the total.  A lane whose DPP
// source is out of its row, or whose row or bank is masked off, keeps the identity.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  auto step = [](uint32_t x, auto ctrl, auto row_mask) {
    const uint32_t y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(0xffffffffu), static_cast<int>(x), decltype(ctrl)::value,
        decltype(row_mask)::value, 0xf, false));
    return x < y ? x : y;
  };
  v = step(v, std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{});   // row_shr:1
  v = step(v, std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{});   // row_shr:2
  v = step(v, std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{});   // row_shr:4
  v = step(v, std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{});   // row_shr:8
  v = step(v, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});   // row_bcast:15
  v = step(v, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});   // row_bcast:31
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__global__ __launch_bounds__(64) void coop_prep_kernel(PrefillArgs a, int flag0, int nflag) {
  int* words = reinterpret_cast<int*>(a.workspace);
  const int t = threadIdx.x;
  if (t == 0) words[0] = 0;
  for (int i = t; i < nflag; i += 64) words[flag0 + i] = 0;
  if (a.lane_units == nullptr) return;
  int32_t* off = const_cast<int32_t*>(a.lane_off);
  int32_t* list = const_cast<int32_t*>(a.lane_units);
  const int H = a.H, U = a.units, N = U / H, L = a.lanes;
  __shared__ int nchs[kPlanMaxSeqs], order[kPlanMaxSeqs], soff[kPlanMaxLanes + 1];
  __shared__ unsigned short lane_of[kPlanMaxUnits], pos_of[kPlanMaxUnits];
  for (int n = t; n < N; n += 64) {
    int ns, hh;
    int64_t bos, eos;
    unit_bounds(a, n * H, ns, hh, bos, eos);
    nchs[n] = static_cast<int>((eos - bos + kChunk - 1) / kChunk);
  }
  __syncthreads();
  for (int n = t; n < N; n += 64) {
    int r = 0;
    for (int m = 0; m < N; ++m) r += (nchs[m] > nchs[n] || (nchs[m] == nchs[n] && m < n)) ? 1 : 0;
    order[r] = n;
  }
  __syncthreads();
  __shared__ uint32_t skey[kPlanMaxLanes], sx[2];
  int load = 0, cnt = 0;   // lane t's chunks and units so far
  for (int r = 0; r < N; ++r) {
    const int n = order[r], c = nchs[n];
    // The sequence's H units weigh the same.  When the H-th smallest lane key is still
    // below the smallest load plus c (with its lane), the greedy rule gives them one
    // each to the H least-loaded lanes in key order: head hh to the lane of rank hh.
    if (H <= L) {
      const uint32_t key = t < L ? (static_cast<uint32_t>(load) << 6) | t : 0xffffffffu;
      if (t < L) skey[t] = key;
      __syncthreads();
      int rank = 0;
      for (int j = 0; j < L; ++j) rank += skey[j] < key ? 1 : 0;
      if (t < L && rank == 0) sx[0] = (static_cast<uint32_t>(load + c) << 6) | t;
      if (t < L && rank == H - 1) sx[1] = key;
      __syncthreads();
      const bool bulk = sx[1] < sx[0];
      if (bulk && t < L && rank < H) {
        lane_of[n * H + rank] = static_cast<unsigned short>(t);
        pos_of[n * H + rank] = static_cast<unsigned short>(cnt);
        ++cnt;
        load += c;
      }
      __syncthreads();   // skey and sx are rewritten for the next sequence
      if (bulk) continue;
    }
    for (int hh = 0; hh < H; ++hh) {
      const uint32_t key = wave_min_u32(t < L ? (static_cast<uint32_t>(load) << 6) | t : 0xffffffffu);
      if (t == static_cast<int>(key & 63)) {
        lane_of[n * H + hh] = static_cast<unsigned short>(t);
        pos_of[n * H + hh] = static_cast<unsigned short>(cnt);
        ++cnt;
        load += c;
      }
    }
  }
  // every unit placed exactly once (the lanes' counts sum to U), else a round-robin plan
  int placed = t < L ? cnt : 0;
  for (int o = 32; o > 0; o >>= 1) placed += __shfl_xor(placed, o);
  if (placed != U) {
    cnt = t < L ? (U - t + L - 1) / L : 0;
    load = 0;
    for (int u = t; u < U; u += 64) {
      lane_of[u] = static_cast<unsigned short>(u % L);
      pos_of[u] = static_cast<unsigned short>(u / L);
    }
    if (t < L)
      for (int u = t; u < U; u += L) load += nchs[u / H];
    __syncthreads();
  }
  // lane offsets: exclusive prefix of the unit counts
  int incl = t < L ? cnt : 0;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (t >= o) incl += y;
  }
  if (t < L) soff[t] = incl - cnt;
  if (t == L - 1) soff[L] = incl;
  __syncthreads();
  for (int i = t; i <= L; i += 64) off[i] = soff[i];
  for (int u = t; u < U; u += 64) list[soff[lane_of[u]] + pos_of[u]] = u;
  if (t < L) list[U + t] = load;   // the lane's total chunks
}

// ====================================================================================
// Launch
// ====================================================================================

// Largest value-tile height each dtype / d_k instantiation of the fused kernel
// supports (LDS budget: fp32 operands are twice the size of bf16 ones).
constexpr int max_bv(bool fp32, int dk) { return fp32 ? (dk == 128 ? 16 : 32) : 64; }
int prefill_max_bv(int dtype, int dk) { return max_bv(dtype == 0, dk); }

template <typename Tin, int DK, int DECAY>
static hipError_t launch_fused_dk(int bv, const PrefillArgs& a, hipStream_t stream) {
  constexpr int kMax = max_bv(sizeof(Tin) == 4, DK);
  const dim3 grid(a.units * a.NV), block(kThreads);
  if constexpr (kMax >= 64) {
    if (bv == 64) {
      hipLaunchKernelGGL((prefill_kernel<Tin, DK, 64, DECAY>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if constexpr (kMax >= 32) {
    if (bv == 32) {
      hipLaunchKernelGGL((prefill_kernel<Tin, DK, 32, DECAY>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_kernel<Tin, DK, 16, DECAY>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <typename Tin, int DECAY>
static hipError_t launch_fused_t(int dk, int bv, const PrefillArgs& a, hipStream_t stream) {
  return dk == 64 ? launch_fused_dk<Tin, 64, DECAY>(bv, a, stream)
                  : launch_fused_dk<Tin, 128, DECAY>(bv, a, stream);
}

template <typename Tin>
static hipError_t launch_fused_d(int dk, int bv, const PrefillArgs& a, hipStream_t stream) {
  if (a.decay == 1) return launch_fused_t<Tin, 1>(dk, bv, a, stream);
  if (a.decay == 2) return launch_fused_t<Tin, 2>(dk, bv, a, stream);
  return launch_fused_t<Tin, 0>(dk, bv, a, stream);
}

// Fused kernel.  bv in {16, 32, 64}, bv <= prefill_max_bv; a.NV = DV / bv.
hipError_t launch_prefill(int dtype, int dk, int bv, const PrefillArgs& a, hipStream_t stream) {
  if (dtype == 1) return launch_fused_d<bf16>(dk, bv, a, stream);
  return launch_fused_d<float>(dk, bv, a, stream);
}

template <int DK, int DECAY>
static hipError_t launch_states_dk(int bv, const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid(a.units * a.NV), block(kThreads);
  if (bv == 64)
    hipLaunchKernelGGL((prefill_kernel<bf16, DK, 64, DECAY, true>), grid, block, 0, stream, a);
  else if (bv == 32)
    hipLaunchKernelGGL((prefill_kernel<bf16, DK, 32, DECAY, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<bf16, DK, 16, DECAY, true>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int DECAY>
static hipError_t launch_states_t(int dk, int bv, const PrefillArgs& a, hipStream_t stream) {
  return dk == 64 ? launch_states_dk<64, DECAY>(bv, a, stream)
                  : launch_states_dk<128, DECAY>(bv, a, stream);
}

// Forward sweep of the backward (bf16): chunk-start states into a.workspace, no o.
hipError_t launch_prefill_states(int dk, int bv, const PrefillArgs& a, hipStream_t stream) {
  if (a.decay == 1) return launch_states_t<1>(dk, bv, a, stream);
  if (a.decay == 2) return launch_states_t<2>(dk, bv, a, stream);
  return launch_states_t<0>(dk, bv, a, stream);
}

size_t prefill_coop_workspace_bytes(int dk, int dv, int lanes, int units, int R, bool plan) {
  if (dk == 64)
    return dv == 64 ? coop_workspace_bytes<64, 64>(lanes, units, R, plan)
                    : coop_workspace_bytes<64, 128>(lanes, units, R, plan);
  return dv == 64 ? coop_workspace_bytes<128, 64>(lanes, units, R, plan)
                  : coop_workspace_bytes<128, 128>(lanes, units, R, plan);
}

template <int DK, int DV, int VBW, int DECAY, bool STATES = false>
static hipError_t launch_wy_k(const PrefillArgs& a, hipStream_t stream) {
  const bool plan = a.lane_units != nullptr;
  const int flag0 = static_cast<int>((kWsHeader + coop_plan_bytes(a.lanes, a.units, plan)) / 4);
  const int nflag = a.lanes * coop_flag_words(a.R);
  hipLaunchKernelGGL(coop_prep_kernel, dim3(1), dim3(64), 0, stream, a, flag0, nflag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillArgs arg = a;
  void* params[] = {&arg};
  const void* kernel =
      reinterpret_cast<const void*>(&prefill_wy_kernel<DK, DV, VBW, DECAY, STATES>);
  const int grid = a.lanes * (a.NC + a.NP);
  // KDA_COOP_LAUNCH=plain: an ordinary dispatch of the same grid when the device holds
  // all of it resident at once (for tools that mishandle cooperative dispatches).  The
  // hand-off waits are bounded either way: a grid that were not resident would abort
  // (NaN outputs, abort word set), never hang.
  const char* mode = std::getenv("KDA_COOP_LAUNCH");
  if (mode != nullptr && std::strcmp(mode, "plain") == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) == hipSuccess &&
        grid <= cus * per_cu) {
      hipLaunchKernelGGL((prefill_wy_kernel<DK, DV, VBW, DECAY, STATES>), dim3(grid),
                         dim3(kThreads), 0, stream, a);
      return hipGetLastError();
    }
  }
  return hipLaunchCooperativeKernel(kernel, dim3(grid), dim3(kThreads), params, 0, stream);
}

template <int DK, int DV, int VBW>
static hipError_t launch_wy_t(const PrefillArgs& a, hipStream_t stream) {
  if (a.decay == 1) return launch_wy_k<DK, DV, VBW, 1>(a, stream);
  if (a.decay == 2) return launch_wy_k<DK, DV, VBW, 2>(a, stream);
  return launch_wy_k<DK, DV, VBW, 0>(a, stream);
}

// Producer/consumer kernel (bf16).  a.NC consumers of a.DV / a.NC value columns
// (4 waves x VBW, VBW in {16, 32}), a.NP producers, a.R ring slots per unit;
// a.workspace holds prefill_coop_workspace_bytes bytes.
hipError_t launch_prefill_coop(int dk, const PrefillArgs& a, hipStream_t stream) {
  const int vbw = a.DV / (4 * a.NC);
  if (dk == 64) {
    if (a.DV == 64) return launch_wy_t<64, 64, 16>(a, stream);
    return vbw == 32 ? launch_wy_t<64, 128, 32>(a, stream) : launch_wy_t<64, 128, 16>(a, stream);
  }
  if (a.DV == 64) return launch_wy_t<128, 64, 16>(a, stream);
  return vbw == 32 ? launch_wy_t<128, 128, 32>(a, stream) : launch_wy_t<128, 128, 16>(a, stream);
}

// Producer/consumer kernel with chunk states (d_k = d_v = 128, a.NC = 2).
hipError_t launch_prefill_coop_states(const PrefillArgs& a, hipStream_t stream) {
  if (a.DV != 128 || a.NC != 2) return hipErrorInvalidValue;
  if (a.decay == 1) return launch_wy_k<128, 128, 16, 1, true>(a, stream);
  if (a.decay == 2) return launch_wy_k<128, 128, 16, 2, true>(a, stream);
  return launch_wy_k<128, 128, 16, 0, true>(a, stream);
}

}  // namespace kda

#if defined(KDA_PHASE_STAMPS)
// Phase sums of the producer/consumer launches since the last kda_phase_clear(), one row
// of kPhaseWords words per workgroup id: words 1..9 ticks per phase, 14 the chunk count,
// 15 the role (consumer index, or 100 + producer index).  Only in a build with
// -DKDA_PHASE_STAMPS (a timing build, not the product).
namespace {
__global__ void phase_clear_kernel() {
  for (int i = threadIdx.x; i < kda::kPhaseWgs * kda::kPhaseWords; i += blockDim.x)
    kda::g_phase[i] = 0;
}
}  // namespace
extern "C" int kda_phase_words(void) { return kda::kPhaseWgs * kda::kPhaseWords; }
extern "C" int kda_phase_clear(void) {
  hipLaunchKernelGGL(phase_clear_kernel, dim3(1), dim3(256), 0, 0);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
extern "C" int kda_phase_read(unsigned int* host) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(kda::g_phase),
                             sizeof(unsigned int) * kda::kPhaseWgs * kda::kPhaseWords) == hipSuccess
             ? 0
             : 1;
}
#endif
