// Backward (training) pass of the chunked KDA prefill on gfx950, bf16 inputs.
//
// The gradient of the chunk algebra of kda_chunk.h.  With H = S^T (d_k x d_v) the
// state at a chunk's start, W = X diag(beta) Kg, U = X diag(beta) V, Kh = k e^{G_n - G}
// and D = Diag(e^{G_n}), one chunk maps
//   E = U - W H,   O = Qg H + M E,   H' = D H + Kh^T E.
// Given dO and dH' (the gradient of the state after the chunk), the reverse step is
//   dE  = Kh dH' + M^T dO                dH = D dH' + Qg^T dO - W^T dE       (the chain)
//   dQg = dO H^T + dM Ki,  dM = lower(dO E^T),   dW = -dE H^T,   dKh = E dH'^T,
//   d e^{G_n}_j = sum_v dH'[j, v] H[j, v],
//   dX  = dE (beta V)^T + dW (beta Kg)^T,   dA = -strict_lower(X^T dX X^T),
//   d(beta V) = X^T dE,   d(beta Kg) = X^T dW + dA Ki,   dKi = dA^T (beta Kg) + dM^T Qg,
// then through Kg = k e^G, Ki = k e^{-G}, Qg = scale q e^G, Kh = k e^{G_n - G} and the
// prefix sums G of g.  The pages tie the chunkwise form to training ("Kimi Delta
// Attention Technical Deep Dive", "Systems and implementation tradeoffs" ->
// "Training"); the derivation is the chain rule through the forward recurrence of
// "Kimi Delta Attention: The Linear Attention Behind Kimi K2 and Qwen3", "How Kimi
// Delta Attention works step by step".
//
// Four launches on one stream:
//   1. forward sweep (prefill_kernel with STATES): the state at every chunk start,
//      bf16, into the workspace;
//   2. the chunk's factors KD, Qg^T, -W^T (MFMA operand fragments), M and e^{G_n} once
//      into the workspace: written by the forward sweep's producers (the
//      producer/consumer kernel), else by bwd_tiles_kernel (one workgroup per chunk and
//      head); then bwd_chain_kernel: per (unit, 16 value rows), the chunks in reverse
//      order, each wave loading its fragments of those tiles into registers a chunk
//      ahead; the chain above only (its value columns are independent), writing dH' of
//      every chunk (bf16) and dL/dS_0;
//   3. bwd_grad_kernel: one workgroup per (chunk, head), all chunks at once; reads H
//      and dH', forms E and dE in 32-wide value slices and accumulates every
//      d_v-contraction in registers, then the chunk-local algebra and the gradients.
// Every product runs on the bf16 MFMA (16x16x32, fp32 accumulation); operands that
// are needed transposed are read with ds_read_b64_tr_b16 (frag_tr).

#include "kda_bwd_launch.h"
#include "kda_chunk.h"
#include "kda_launch.h"
#include "kda_tiles.h"
#include "kda_wy.h"

namespace kda {

static_assert(ChainTiles<64>::kBytes == chain_tile_bytes(64) &&
                  ChainTiles<128>::kBytes == chain_tile_bytes(128),
              "host and device chunk-tile sizes agree");

using MB = Mfma<bf16>;

__device__ __forceinline__ bf16x8 frow(const bf16* base, int ld, int row0, int k0, int lane) {
  return frag_rows<MB>(base, ld, row0, k0, lane);
}

// ====================================================================================
// Chunk tiles of the reverse chain
// ====================================================================================

// Sequence and chunk of a chunk slot (see chunk_slot_base); false for an unused slot.
__device__ __forceinline__ bool slot_chunk(const BwdArgs& a, int64_t slot, int& n_seq,
                                           int64_t& bos, int64_t& eos, int& c) {
  auto bos_of = [&](int n) -> int64_t {
    return a.cu_seqlens ? static_cast<int64_t>(a.cu_seqlens[n]) : static_cast<int64_t>(n) * a.T;
  };
  int lo = 0, hi = a.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_slot_base(mid, bos_of(mid)) <= slot) lo = mid; else hi = mid - 1;
  }
  n_seq = lo;
  bos = bos_of(lo);
  eos = a.cu_seqlens ? static_cast<int64_t>(a.cu_seqlens[lo + 1]) : bos + a.T;
  const int64_t cc = slot - chunk_slot_base(lo, bos);
  c = static_cast<int>(cc);
  return cc >= 0 && cc * kChunk < eos - bos;
}

// One workgroup per (chunk slot, head): the chunk's factors (as the forward computes
// them), copied to the workspace.
template <int DK, int DECAY>
__global__ __launch_bounds__(kThreads, 1) void bwd_tiles_kernel(BwdArgs a) {
  using CP = ChunkProducer<bf16, DK, false>;
  using CL = ChunkLayout<bf16, DK, false>;
  using TL = ChainTiles<DK>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[CL::kBytes];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % a.H;
  const int64_t slot = blockIdx.x / a.H;
  int n_seq, c;
  int64_t bos, eos;
  if (!slot_chunk(a, slot, n_seq, bos, eos, c)) return;   // uniform over the workgroup
  const int64_t c0 = bos + int64_t(c) * kChunk;
  const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
  CP cp;
  cp.init(smem, static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k), a.g, a.beta, a.H,
          h, a.scale, tid, wave, a.flags);
  cp.template load<DECAY>(c0, n);
  cp.template factors<DECAY>(n, false, 0, 0);
  cp.products();
  cp.inverse();   // ends with a barrier
  // -W = -X diag(beta) Kg for token block `wave` into the A area (dead after the
  // inverse), bf16 rows with the stride of the other tiles
  constexpr int LDK = CL::LDK, LDC = CL::LDC, NKB = DK / 16;
  static_assert(LDK == DK + 8 && LDC == kChunk + 8, "tile row strides");
  static_assert(size_t(kChunk) * LDK * 2 <= CL::oX - CL::oA, "W tile fits the A area");
  bf16* sW = reinterpret_cast<bf16*>(smem + CL::oA);
  {
    const int lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    f32x4 acc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < 16 * (wave + 1); kk += 32) {   // X is lower triangular
      bf16x8 xa = frow(cp.sTm, LDC, 16 * wave, kk, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        xa[e] = static_cast<bf16>(static_cast<float>(xa[e]) * cp.sBeta[kk + 8 * lq + e]);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        acc[kb] = mma_bf16(xa, frag_tr(cp.sKg, LDK, kk, 16 * kb, lane), acc[kb]);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sW[(16 * wave + 4 * lq + i) * LDK + 16 * kb + lr] = static_cast<bf16>(-acc[kb][i]);
  }
  lds_barrier();
  unsigned char* dst = static_cast<unsigned char*>(a.tiles) + (slot * a.H + h) * TL::kBytes;
  const int lane = tid & 63;
  store_kd_frags<DK>(dst, cp.sKi, LDK, cp.sEgn, true, wave, lane);   // KD = Ki Diag(e^{G_n})
  store_tr_frags<DK>(dst + TL::oQT, cp.sQg, LDK, wave, lane);
  store_tr_frags<DK>(dst + TL::oWT, sW, LDK, wave, lane);
  for (int q = tid; q < TL::PC; q += kThreads)
    __builtin_nontemporal_store(*reinterpret_cast<const bf16x8*>(cp.sM + (q / 8) * LDC + 8 * (q % 8)),
                                reinterpret_cast<bf16x8*>(dst + TL::oM + 16 * size_t(q)));
  store_egn<DK>(dst, cp.sEgn, tid);
}

// ====================================================================================
// Reverse chain
// ====================================================================================

template <int DK, int BV>
struct ChainLayout {
  static constexpr int LDK = DK + 8, LDC = kChunk + 8;
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t tC = size_t(kChunk) * LDC * 2;
  static constexpr size_t oM = 0;                                      // two M tiles [64][LDC]
  static constexpr size_t oP = 2 * tC;                                 // dH'^T [BV][LDK]
  static constexpr size_t oDOT = al(oP + size_t(BV) * LDK * 2);       // [BV][LDC] each
  static constexpr size_t oDET = al(oDOT + size_t(BV) * LDC * 2);
  static constexpr size_t oTouch = al(oDET + size_t(BV) * LDC * 2);   // 4 B per thread, never read
  static constexpr size_t kBytes = oTouch + size_t(kThreads) * 4;
  static_assert(kBytes <= 160 * 1024, "LDS budget exceeded");
};

// Per (unit, BV value rows), the chunks in reverse order.  Each wave loads the operand
// fragments it uses straight from the chunk's tiles into registers, a chunk ahead: its
// token block of KD (for dE), its key blocks of Qg^T, -W^T and e^{G_n} (for dH).  M,
// read transposed, goes through one of two LDS buffers filled a chunk ahead.
template <int DK, int BV>
__global__ __launch_bounds__(kThreads, 1) void bwd_chain_kernel(BwdArgs a) {
  using CL = ChainLayout<DK, BV>;
  using TL = ChainTiles<DK>;
  using ST = StateTiles<DK, BV>;
  constexpr int LDK = CL::LDK, LDC = CL::LDC, NVB = BV / 16, NKS = DK / 32;
  constexpr int MPT = TL::PC / kThreads;   // M pieces per thread
  static_assert(MPT * kThreads == TL::PC, "M pieces");

  __shared__ __attribute__((aligned(16))) unsigned char smem[CL::kBytes];
  bf16* sP = reinterpret_cast<bf16*>(smem + CL::oP);
  bf16* sDOT = reinterpret_cast<bf16*>(smem + CL::oDOT);
  bf16* sDET = reinterpret_cast<bf16*>(smem + CL::oDET);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  int unit, vt, n_seq, h;
  int64_t bos, eos;
  unit_role(blockIdx.x, a.NV, a.units, a.xcd_remap, unit, vt);
  unit_bounds(a, unit, n_seq, h, bos, eos);
  const int v0 = vt * BV;
  const bf16* dout = static_cast<const bf16*>(a.dout);
  bf16* dstates = static_cast<bf16*>(a.dstates);
  const unsigned char* tiles = static_cast<const unsigned char*>(a.tiles);

  f32x4 sacc[ST::NST];   // dH^T tiles of this value tile (rows = key), fp32
  const int64_t st_base = (static_cast<int64_t>(n_seq) * a.H + h) * a.DV * DK;
  load_state<DK, BV, LDK>(sacc, a.dfinal_state, st_base, v0, sP, wave, lane);

  const int nch = static_cast<int>((eos - bos + kChunk - 1) / kChunk);
  const int64_t slot0 = chunk_slot_base(n_seq, bos);
  auto tile = [&](int c) { return tiles + ((slot0 + c) * a.H + h) * TL::kBytes; };

  // One chunk's operands in registers.  Each set is requested for the previous chunk
  // right after its last use in this one, so it has a whole chunk to arrive and the
  // requests are spread over the chunk.
  bf16x8 kd[NKS];                          // KD row 16 wave + l % 16, keys 32 s + 8 (l / 16) ..
  bf16x8 qt[ST::NST][2], wt[ST::NST][2];   // Qg^T, -W^T key 16 kb + l % 16, tokens 32 u + 8 (l / 16) ..
  f32x4 eg[ST::NST];                       // e^{G_n} of keys 16 kb + 4 (l / 16) .. +3
  u32x4 mp[MPT];                           // M pieces on their way to LDS
  auto load_kd = [&](int c) {
    const unsigned char* tk = tile(c) + TL::oKD + 1024 * size_t(wave * NKS) + 16 * lane;
#pragma unroll
    for (int s = 0; s < NKS; ++s) kd[s] = *reinterpret_cast<const bf16x8*>(tk + 1024 * s);
  };
  auto load_dh = [&](int c) {
    const unsigned char* t = tile(c);
#pragma unroll
    for (int s = 0; s < ST::NST; ++s) {
      const int kb = ST::kb(wave, s);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const size_t q = 1024 * size_t(2 * kb + u) + 16 * lane;
        qt[s][u] = *reinterpret_cast<const bf16x8*>(t + TL::oQT + q);
        wt[s][u] = *reinterpret_cast<const bf16x8*>(t + TL::oWT + q);
      }
      eg[s] = *reinterpret_cast<const f32x4*>(t + TL::oE + (16 * kb + 4 * lq) * 4);
    }
  };
  auto load_m = [&](int c) {
    const unsigned char* t = tile(c) + TL::oM;
#pragma unroll
    for (int i = 0; i < MPT; ++i)
      mp[i] = *reinterpret_cast<const u32x4*>(t + 16 * size_t(tid + i * kThreads));
  };
  auto deposit_m = [&](int buf) {
    bf16* sMb = reinterpret_cast<bf16*>(smem + CL::oM + buf * CL::tC);
#pragma unroll
    for (int i = 0; i < MPT; ++i) {
      const int q = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(sMb + (q / 8) * LDC + 8 * (q % 8)) = mp[i];
    }
  };
  // Chunk c's tiles into L2 two chunks ahead of their use: one 4-byte read per 128-byte
  // line, issued after the chunk's other reads (no wait for those covers these) and
  // consumed at the chunk's end, a whole chunk later.
  constexpr int kLines = static_cast<int>((TL::kBytes + 127) / 128);
  constexpr int NT = (kLines + 4 * 64 - 1) / (4 * 64);   // reads per lane
  uint32_t tw[NT], tacc = 0;
  auto touch = [&](int c) {
    const uint32_t* base = reinterpret_cast<const uint32_t*>(tile(c));
#pragma unroll
    for (int j = 0; j < NT; ++j) tw[j] = base[32 * min(64 * (4 * j + wave) + lane, kLines - 1)];
  };
  ValueRegs<bf16, NVB> dr;   // dO rows of the chunk, accumulator layout
  if (nch > 0) {
    // the loop's own order (M, dO, KD, the dH operands): the compiler's wait at the loop
    // top for dO then never covers the later reads
    const int64_t cl = bos + int64_t(nch - 1) * kChunk;
    load_m(nch - 1);
    dr.load(dout, cl, static_cast<int>(eos - cl), a.H, h, a.DV, v0, wave, lane);
    load_kd(nch - 1);
    load_dh(nch - 1);
    deposit_m(0);
  }
  lds_barrier();
  const int k0m = (16 * wave) & ~31;   // first K step that meets a triangular row block

  for (int c = nch - 1; c >= 0; --c) {
    const int cur = (nch - 1 - c) & 1;
    const bf16* sM = reinterpret_cast<const bf16*>(smem + CL::oM + cur * CL::tC);
    const int64_t c0 = bos + int64_t(c) * kChunk;
    const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
    // the chunk whose operands are loaded during this one: the previous chunk in token
    // order (always full), or the first one again at the end (in bounds, unused)
    const int cp = c > 0 ? c - 1 : 0;
    // dO^T of this chunk (its rows were requested a chunk ago)
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = 16 * wave + 4 * lq + i < n ? dr.f32(vb, i) : 0.f;
      store4(sDOT + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, x);
    }
    load_m(cp);
    // dL/d(state after chunk c)
    store_state_bf16<DK, BV>(sacc, dstates, ((slot0 + c) * a.H + h) * a.DV * DK, v0, wave,
                             lane);
    // dH', the operand of dE
#pragma unroll
    for (int s = 0; s < ST::NST; ++s) {
      const int kb = ST::kb(wave, s), vb = ST::vb(s);
      store4(sP + (16 * vb + lr) * LDK + 16 * kb + 4 * lq, sacc[s]);
    }
    dr.load(dout, bos + int64_t(cp) * kChunk, static_cast<int>(min(eos - bos - int64_t(cp) * kChunk,
                                                                   static_cast<int64_t>(kChunk))),
            a.H, h, a.DV, v0, wave, lane);
    touch(c > 1 ? c - 2 : 0);
    lds_barrier();

    // dE = KD dH' + M^T dO for token block `wave` -> dE^T
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s) acc = mma_bf16(kd[s], frow(sP, LDK, 16 * vb, 32 * s, lane), acc);
      for (int kk = k0m; kk < kChunk; kk += 32)
        acc = mma_bf16(frag_tr(sM, LDC, kk, 16 * wave, lane), frow(sDOT, LDC, 16 * vb, kk, lane),
                       acc);
      store4(sDET + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, acc);
    }
    load_kd(cp);
    lds_barrier();

    // dH = D dH' + Qg^T dO - W^T dE
#pragma unroll
    for (int s = 0; s < ST::NST; ++s) {
      const int vb = ST::vb(s);
      f32x4 acc = sacc[s] * eg[s];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        acc = mma_bf16(qt[s][u], frow(sDOT, LDC, 16 * vb, 32 * u, lane), acc);
        acc = mma_bf16(wt[s][u], frow(sDET, LDC, 16 * vb, 32 * u, lane), acc);
      }
      sacc[s] = acc;
    }
    load_dh(cp);
    deposit_m(cur ^ 1);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < NT; ++j) tacc ^= tw[j];
  }
  // the touched words end in a scratch corner of LDS (volatile: the reads stay)
  *reinterpret_cast<volatile uint32_t*>(smem + CL::oTouch + 4 * tid) = tacc;
  if (a.dinitial_state) store_state<DK, BV>(sacc, a.dinitial_state, st_base, v0, wave, lane);
}

// ====================================================================================
// Chunk-parallel gradients
// ====================================================================================

#if defined(KDA_PHASE_STAMPS)
// Timing build only: per (chunk, head) item, the s_memtime ticks of the gradient
// kernel's phases (words 1..8: loads and factors, A and M, inverse, value slices,
// chunk-local algebra, k/q deposit, per-element gradients, dq/dk/dg output; words 10..13
// the value slices' staging, R'/dE, E/dv and d_v contractions summed over slices; word
// 15 = 1 for a written row), read with kda_grad_phase_read().
constexpr int kGradPhaseItems = 40000, kGradPhaseWords = 16;
__device__ unsigned int g_grad_phase[kGradPhaseItems * kGradPhaseWords];
#endif

template <int DK>
struct GradLayout {
  using CL = ChunkLayout<bf16, DK, false>;
  static constexpr int LDK = CL::LDK, LDC = CL::LDC;
  static constexpr int LDEG = ChunkProducer<bf16, DK, false>::LDEG;
  static constexpr int VS = 32;                                   // value slice
  static constexpr size_t oEG = CL::kBytes;                       // fp32 e^{G} [DK][LDEG]
  static constexpr size_t kBytes = CL::al(oEG + size_t(DK) * LDEG * 4);
  static constexpr size_t kLds = 160 * 1024;
  // area 1: A and the fp32 inverse (dead after the inverse); area 2: the rest of LDS
  static constexpr size_t a1 = CL::oA, a1end = CL::oScr;
  static constexpr size_t a2 = kBytes, a2end = kLds;
  static constexpr size_t tV = size_t(VS) * LDK * 2;              // [VS][LDK] bf16
  static constexpr size_t tT = size_t(VS) * LDC * 2;              // [VS][LDC] bf16
  static constexpr int LDV = VS + 8;                              // [64][LDV] bf16 rows
  static constexpr size_t tR = size_t(kChunk) * LDV * 2;
  static constexpr size_t tC = size_t(kChunk) * LDC * 2;          // [64][LDC] bf16
  static constexpr size_t tW = size_t(DK) * LDC * 2;              // [DK][LDC] bf16
  // value-slice phase
  static constexpr size_t oH = a1, oDH = a1 + tV, oP = a1 + 2 * tV, oRT = a1 + 3 * tV;
  static constexpr size_t oET = a2, oDET = a2 + tT, oDO = a2 + 2 * tT, oV = oDO + tR;
  static constexpr size_t oDV = oRT + tT;                         // dv slice [64][VS] bf16
  static_assert(oDV + size_t(kChunk) * VS * 2 <= a1end && oV + tR <= a2end,
                "value-slice tiles overflow");
  // chunk-local phase
  static constexpr size_t oDWT = a1, oDMT = a1 + tW;
  static constexpr size_t oCC1 = a2, oCC2 = a2 + tC, oCC3 = CL::oM;
  static_assert(oDMT + tC <= a1end && oCC2 + tC <= a2end, "chunk tiles overflow");
  // gradients: raw k, q tiles (then dk, dq) and the reduction scratch
  static constexpr size_t tK = size_t(kChunk) * LDK * 2;
  static constexpr size_t oK = a1, oQ = a1 + tK;
  static constexpr size_t oRed = a2;                              // fp32 [12][DK]
  static constexpr int LDG = DK + 8;                              // dg rows (fp32), in area 1
  static_assert(oQ + tK <= a1end, "k/q tiles overflow");
  static_assert(a1 + size_t(kChunk) * LDG * 4 <= a1end, "dg tile overflow");
  static_assert(oRed + size_t(12) * DK * 4 <= a2end, "reduction overflow");
  static_assert(kBytes <= kLds, "LDS budget exceeded");
};

template <int DK, int DV, int DECAY>
__global__ __launch_bounds__(kThreads, 1) void bwd_grad_kernel(BwdArgs a) {
  using CP = ChunkProducer<bf16, DK, false>;
  using GL = GradLayout<DK>;
  constexpr int LDK = GL::LDK, LDC = GL::LDC, LDEG = GL::LDEG, VS = GL::VS;
  constexpr int NKB = DK / 16;

  __shared__ __attribute__((aligned(16))) unsigned char smem[GL::kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;

  const int h = blockIdx.x % a.H;
  const int64_t slot = blockIdx.x / a.H;
  int n_seq, c;
  int64_t bos, eos;
  if (!slot_chunk(a, slot, n_seq, bos, eos, c)) return;   // uniform over the workgroup
  const int64_t c0 = bos + int64_t(c) * kChunk;
  const int n = static_cast<int>(min(eos - c0, static_cast<int64_t>(kChunk)));
  const int64_t sbase = ((slot * a.H + h) * a.DV) * DK;
  KDA_PHASE(unsigned long long gt_[9]; unsigned gs_[4] = {0, 0, 0, 0}; gt_[0] = __builtin_amdgcn_s_memtime();)
  const bf16* states = static_cast<const bf16*>(a.states) + sbase;
  const bf16* dstates = static_cast<const bf16*>(a.dstates) + sbase;
  const bf16* vin = static_cast<const bf16*>(a.v);
  const bf16* dout = static_cast<const bf16*>(a.dout);
  const bf16* kin = static_cast<const bf16*>(a.k);
  const bf16* qin = static_cast<const bf16*>(a.q);
  bf16* dvout = static_cast<bf16*>(a.dv);
  const uint32_t rowV = static_cast<uint32_t>(a.H) * DV;
  const uint32_t rowK = static_cast<uint32_t>(a.H) * DK;

  // value slices of H, dH', V and dO: each slice's pieces are requested into registers
  // one slice ahead (the first while the chunk's factors are computed)
  constexpr int HPT = VS * DK / 8 / kThreads;   // 16-byte pieces of H (and of dH') per thread
  static_assert(HPT * kThreads * 8 == VS * DK && kChunk * VS / 8 == kThreads, "slice pieces");
  bf16x8 ph[HPT], pdh[HPT], pv, pdo;
  auto fetch_slice = [&](int vs) {
    const int v0 = vs * VS;
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
      ph[i] = *reinterpret_cast<const bf16x8*>(states + int64_t(v0 + r) * DK + c8);
      pdh[i] = *reinterpret_cast<const bf16x8*>(dstates + int64_t(v0 + r) * DK + c8);
    }
    const int r = tid / (VS / 8), c8 = 8 * (tid % (VS / 8));
    pv = bf16x8{};
    pdo = bf16x8{};
    if (r < n) {
      const int64_t o = (c0 + r) * rowV + int64_t(h) * DV + v0 + c8;
      pv = *reinterpret_cast<const bf16x8*>(vin + o);
      pdo = *reinterpret_cast<const bf16x8*>(dout + o);
    }
  };
  fetch_slice(0);

  CP cp;
  cp.init(smem, qin, kin, a.g, a.beta, a.H, h, a.scale, tid, wave, a.flags);
  cp.sEG = reinterpret_cast<float*>(smem + GL::oEG);
  cp.template load<DECAY>(c0, n);
  cp.template factors<DECAY, true>(n, false, 0, 0);
  KDA_PHASE(gt_[1] = __builtin_amdgcn_s_memtime();)
  cp.products();
  KDA_PHASE(gt_[2] = __builtin_amdgcn_s_memtime();)
  cp.inverse();
  KDA_PHASE(gt_[3] = __builtin_amdgcn_s_memtime();)

  const int k0m = (16 * wave) & ~31;
  const int kend = 16 * (wave + 1);
  const f32x4 bt = *reinterpret_cast<const f32x4*>(cp.sBeta + 16 * wave + 4 * lq);

  // ---- value slices: E, dE, and every contraction over d_v ----------------------------
  bf16* sH = reinterpret_cast<bf16*>(smem + GL::oH);
  bf16* sDH = reinterpret_cast<bf16*>(smem + GL::oDH);
  bf16* sP = reinterpret_cast<bf16*>(smem + GL::oP);
  bf16* sRT = reinterpret_cast<bf16*>(smem + GL::oRT);
  bf16* sET = reinterpret_cast<bf16*>(smem + GL::oET);
  bf16* sDET = reinterpret_cast<bf16*>(smem + GL::oDET);
  bf16* sDO = reinterpret_cast<bf16*>(smem + GL::oDO);   // dO slice [64][LDV], token rows
  bf16* sV = reinterpret_cast<bf16*>(smem + GL::oV);     // V slice [64][LDV]
  bf16* sDV = reinterpret_cast<bf16*>(smem + GL::oDV);   // dv slice [64][VS]
  constexpr int LDV = GL::LDV;

  f32x4 dQg[NKB], dWn[NKB], dKh[NKB], dM[4], dXU[4];
#pragma unroll
  for (int i = 0; i < NKB; ++i) dQg[i] = dWn[i] = dKh[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) dM[i] = dXU[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 dbu = f32x4{0.f, 0.f, 0.f, 0.f};   // sum_v d(beta V) V for this lane's rows
  float ddk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // d e^{G_n} of this thread's keys

  // e^{G_n} of this thread's eight keys: the same eight in each of its slice pieces
  static_assert(kThreads % (DK / 8) == 0, "one key octet per thread");
  float egk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) egk[e] = cp.sEgn[8 * (tid % (DK / 8)) + e];

  for (int vs = 0; vs < DV / VS; ++vs) {
    const int v0 = vs * VS;
    KDA_PHASE(unsigned long long u0_ = __builtin_amdgcn_s_memtime(), u1_;)
    // H, dH' (and P = D dH') slices [VS][DK]; V and dO slices [64][VS]; d e^{G_n} partial
    // sums of this thread's eight keys from the same registers
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
      *reinterpret_cast<bf16x8*>(sH + r * LDK + c8) = ph[i];
      *reinterpret_cast<bf16x8*>(sDH + r * LDK + c8) = pdh[i];
      bf16x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dh = static_cast<float>(pdh[i][e]);
        p[e] = static_cast<bf16>(dh * egk[e]);
        ddk[e] += dh * static_cast<float>(ph[i][e]);
      }
      *reinterpret_cast<bf16x8*>(sP + r * LDK + c8) = p;
    }
    {
      const int r = tid / (VS / 8), c8 = 8 * (tid % (VS / 8));
      *reinterpret_cast<bf16x8*>(sV + r * LDV + c8) = pv;
      *reinterpret_cast<bf16x8*>(sDO + r * LDV + c8) = pdo;
    }
    if (vs + 1 < DV / VS) fetch_slice(vs + 1);
    lds_barrier();
    KDA_PHASE(u1_ = __builtin_amdgcn_s_memtime(); gs_[0] += unsigned(u1_ - u0_); u0_ = u1_;)
    f32x4 vreg[VS / 16];   // V in accumulator layout (rows of this wave)
#pragma unroll
    for (int vb = 0; vb < VS / 16; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vreg[vb][i] = static_cast<float>(sV[(16 * wave + 4 * lq + i) * LDV + 16 * vb + lr]);

    // R' = beta (V - Kg H) -> R'^T;  dE = Ki P + M^T dO -> dE^T
    {
      f32x4 acc[VS / 16], de[VS / 16];
#pragma unroll
      for (int vb = 0; vb < VS / 16; ++vb) acc[vb] = de[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < DK; kk += 32) {
        const bf16x8 aK = frow(cp.sKg, LDK, 16 * wave, kk, lane);
        const bf16x8 aKi = frow(cp.sKi, LDK, 16 * wave, kk, lane);
#pragma unroll
        for (int vb = 0; vb < VS / 16; ++vb) {
          acc[vb] = mma_bf16(aK, frow(sH, LDK, 16 * vb, kk, lane), acc[vb]);
          de[vb] = mma_bf16(aKi, frow(sP, LDK, 16 * vb, kk, lane), de[vb]);
        }
      }
      for (int kk = k0m; kk < kChunk; kk += 32) {
        const bf16x8 aM = frag_tr(cp.sM, LDC, kk, 16 * wave, lane);
#pragma unroll
        for (int vb = 0; vb < VS / 16; ++vb)
          de[vb] = mma_bf16(aM, frag_tr(sDO, LDV, kk, 16 * vb, lane), de[vb]);
      }
#pragma unroll
      for (int vb = 0; vb < VS / 16; ++vb) {
        store4(sRT + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, bt * (vreg[vb] - acc[vb]));
        store4(sDET + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, de[vb]);
      }
    }
    lds_barrier();
    KDA_PHASE(u1_ = __builtin_amdgcn_s_memtime(); gs_[1] += unsigned(u1_ - u0_); u0_ = u1_;)

    // E = X R' -> E^T;  d(beta V) = X^T dE -> dv, and its dot with V
    {
      f32x4 e[VS / 16], dbv[VS / 16];
#pragma unroll
      for (int vb = 0; vb < VS / 16; ++vb) e[vb] = dbv[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kk = 0; kk < kend; kk += 32) {
        const bf16x8 aT = frow(cp.sTm, LDC, 16 * wave, kk, lane);
#pragma unroll
        for (int vb = 0; vb < VS / 16; ++vb)
          e[vb] = mma_bf16(aT, frow(sRT, LDC, 16 * vb, kk, lane), e[vb]);
      }
      for (int kk = k0m; kk < kChunk; kk += 32) {
        const bf16x8 aTt = frag_tr(cp.sTm, LDC, kk, 16 * wave, lane);
#pragma unroll
        for (int vb = 0; vb < VS / 16; ++vb)
          dbv[vb] = mma_bf16(aTt, frow(sDET, LDC, 16 * vb, kk, lane), dbv[vb]);
      }
#pragma unroll
      for (int vb = 0; vb < VS / 16; ++vb) {
        store4(sET + (16 * vb + lr) * LDC + 16 * wave + 4 * lq, e[vb]);
        dbu += dbv[vb] * vreg[vb];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sDV[(16 * wave + 4 * lq + i) * VS + 16 * vb + lr] = static_cast<bf16>(bt[i] * dbv[vb][i]);
      }
    }
    lds_barrier();
    KDA_PHASE(u1_ = __builtin_amdgcn_s_memtime(); gs_[2] += unsigned(u1_ - u0_); u0_ = u1_;)

    // this slice's dv rows leave as 16-byte pieces (one per thread)
    {
      const int r = tid / (VS / 8), c8 = 8 * (tid % (VS / 8));
      if (r < n)
        *reinterpret_cast<bf16x8*>(dvout + (c0 + r) * rowV + int64_t(h) * DV + v0 + c8) =
            *reinterpret_cast<const bf16x8*>(sDV + r * VS + c8);
    }
    // contractions over this slice's values (K = 32 = one MFMA step)
    {
      const bf16x8 aDO = frow(sDO, LDV, 16 * wave, 0, lane);
      const bf16x8 aDE = frag_tr(sDET, LDC, 0, 16 * wave, lane);
      const bf16x8 aE = frag_tr(sET, LDC, 0, 16 * wave, lane);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 bH = frag_tr(sH, LDK, 0, 16 * kb, lane);
        dQg[kb] = mma_bf16(aDO, bH, dQg[kb]);
        dWn[kb] = mma_bf16(aDE, bH, dWn[kb]);
        dKh[kb] = mma_bf16(aE, frag_tr(sDH, LDK, 0, 16 * kb, lane), dKh[kb]);
      }
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        dM[sb] = mma_bf16(aDO, frag_tr(sET, LDC, 0, 16 * sb, lane), dM[sb]);
        dXU[sb] = mma_bf16(aDE, frow(sV, LDV, 16 * sb, 0, lane), dXU[sb]);
      }
    }
    lds_barrier();
    KDA_PHASE(u1_ = __builtin_amdgcn_s_memtime(); gs_[3] += unsigned(u1_ - u0_);)
  }

  // ---- chunk-local algebra -------------------------------------------------------------
  // Every slice read has landed (and the dv stores are acknowledged): saying so lets the
  // compiler count the reads below exactly instead of waiting for all of them at the
  // first reuse of a slice register.
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  KDA_PHASE(gt_[4] = __builtin_amdgcn_s_memtime();)
  // the chunk's raw k and q rows, requested now for the gradients at the end
  constexpr int KPT2 = kChunk * DK / 8 / kThreads;
  bf16x8 pk[KPT2], pq[KPT2];
#pragma unroll
  for (int i = 0; i < KPT2; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
    pk[i] = bf16x8{};
    pq[i] = bf16x8{};
    if (r < n) {
      const int64_t o = (c0 + r) * rowK + int64_t(h) * DK + c8;
      pk[i] = *reinterpret_cast<const bf16x8*>(kin + o);
      pq[i] = *reinterpret_cast<const bf16x8*>(qin + o);
    }
  }
  bf16* sDWT = reinterpret_cast<bf16*>(smem + GL::oDWT);   // dW^T [DK][64]
  bf16* sDMT = reinterpret_cast<bf16*>(smem + GL::oDMT);   // dM^T [64][64]
  bf16* sC1 = reinterpret_cast<bf16*>(smem + GL::oCC1);
  bf16* sC2 = reinterpret_cast<bf16*>(smem + GL::oCC2);
  bf16* sC3 = reinterpret_cast<bf16*>(smem + GL::oCC3);
  // dW = -dE H^T (transposed), dM = lower(dO E^T) (transposed)
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    store4(sDWT + (16 * kb + lr) * LDC + 16 * wave + 4 * lq, -dWn[kb]);
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 16 * sb + lr <= 16 * wave + 4 * lq + i ? dM[sb][i] : 0.f;
    store4(sDMT + (16 * sb + lr) * LDC + 16 * wave + 4 * lq, x);
  }
  lds_barrier();

  // dX = (dE V^T + dW Kg^T) Diag(beta), strictly lower -> dX^T (sC1)
#pragma unroll
  for (int kk = 0; kk < DK; kk += 32) {
    const bf16x8 aW = frag_tr(sDWT, LDC, kk, 16 * wave, lane);
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
      dXU[sb] = mma_bf16(aW, frow(cp.sKg, LDK, 16 * sb, kk, lane), dXU[sb]);
  }
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const f32x4 acc = dXU[sb];
    const float bs = cp.sBeta[16 * sb + lr];
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 16 * sb + lr < 16 * wave + 4 * lq + i ? acc[i] * bs : 0.f;
    store4(sC1 + (16 * sb + lr) * LDC + 16 * wave + 4 * lq, x);
  }
  lds_barrier();

  // Y = dX X^T -> Y^T (sC2)
  {
    f32x4 acc[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < kend; kk += 32) {
      const bf16x8 aX = frag_tr(sC1, LDC, kk, 16 * wave, lane);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        acc[jb] = mma_bf16(aX, frow(cp.sTm, LDC, 16 * jb, kk, lane), acc[jb]);
    }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) store4(sC2 + (16 * jb + lr) * LDC + 16 * wave + 4 * lq, acc[jb]);
  }
  lds_barrier();

  // dA = -strict_lower(X^T Y) -> dA^T (sC1) and (Diag(beta) dA)^T (sC3)
  f32x4 dAacc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) dAacc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = k0m; kk < kChunk; kk += 32) {
    const bf16x8 aXt = frag_tr(cp.sTm, LDC, kk, 16 * wave, lane);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) dAacc[jb] = mma_bf16(aXt, frow(sC2, LDC, 16 * jb, kk, lane), dAacc[jb]);
  }
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const f32x4 acc = dAacc[jb];
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 16 * jb + lr < 16 * wave + 4 * lq + i ? -acc[i] : 0.f;
    store4(sC1 + (16 * jb + lr) * LDC + 16 * wave + 4 * lq, x);
    store4(sC3 + (16 * jb + lr) * LDC + 16 * wave + 4 * lq, x * bt);
  }
  lds_barrier();

  // d(beta Kg) = X^T dW + dA Ki;  dKi = dA^T (beta Kg) + dM^T Qg;  dQg += dM Ki
  // (the A operands depend on the K step only: loaded once per step for all key blocks)
  f32x4 dBk[NKB], dKi[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) dBk[kb] = dKi[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kk = k0m; kk < kChunk; kk += 32) {
    const bf16x8 aXt = frag_tr(cp.sTm, LDC, kk, 16 * wave, lane);
    const bf16x8 aAb = frow(sC3, LDC, 16 * wave, kk, lane);
    const bf16x8 aMt = frow(sDMT, LDC, 16 * wave, kk, lane);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      dBk[kb] = mma_bf16(aXt, frow(sDWT, LDC, 16 * kb, kk, lane), dBk[kb]);
      dKi[kb] = mma_bf16(aAb, frag_tr(cp.sKg, LDK, kk, 16 * kb, lane), dKi[kb]);
      dKi[kb] = mma_bf16(aMt, frag_tr(cp.sQg, LDK, kk, 16 * kb, lane), dKi[kb]);
    }
  }
  for (int kk = 0; kk < kend; kk += 32) {
    const bf16x8 aA = frag_tr(sC1, LDC, kk, 16 * wave, lane);
    const bf16x8 aM = frag_tr(sDMT, LDC, kk, 16 * wave, lane);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 bKi = frag_tr(cp.sKi, LDK, kk, 16 * kb, lane);
      dBk[kb] = mma_bf16(aA, bKi, dBk[kb]);
      dQg[kb] = mma_bf16(aM, bKi, dQg[kb]);
    }
  }
  lds_barrier();
  KDA_PHASE(gt_[5] = __builtin_amdgcn_s_memtime();)

  // ---- gradients of k, q, beta, g ----------------------------------------------------
  // the chunk's raw k and q (bf16, exact) into LDS; each element's gradient then
  // replaces it in place (one owner per element), and the rows leave as 16-byte stores
  bf16* sK = reinterpret_cast<bf16*>(smem + GL::oK);
  bf16* sQ = reinterpret_cast<bf16*>(smem + GL::oQ);
#pragma unroll
  for (int i = 0; i < KPT2; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
    *reinterpret_cast<bf16x8*>(sK + r * LDK + c8) = pk[i];
    *reinterpret_cast<bf16x8*>(sQ + r * LDK + c8) = pq[i];
  }
  lds_barrier();
  KDA_PHASE(gt_[6] = __builtin_amdgcn_s_memtime();)

  // per element: dk, dq, and dL/dG = dKg Kg + dQg Qg - dKi Ki - dKh Kh, summed over the
  // rows at or below it within this wave's token block (suffix); the block totals, the
  // dG_n partials and the d e^{G_n} partials go to LDS
  float* sRed = reinterpret_cast<float*>(smem + GL::oRed);   // [4][DK] [4][DK] [4][DK]
  f32x4 dbk = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 gm[NKB];
  // raw keys: the factors used the unit key bf16(k / n), n = sqrt(|k|^2 + eps) per row;
  // its gradient dk^ is carried back to k as (dk^ - k^ (k^ . dk^)) / n
  const bool norm_k = (a.flags & kNormK) != 0;
  f32x4 rn = f32x4{1.f, 1.f, 1.f, 1.f}, kdot = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 dkh[NKB];
  if (norm_k) {
    f32x4 ss = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float kf = static_cast<float>(sK[(16 * wave + 4 * lq + i) * LDK + 16 * kb + lr]);
        ss[i] += kf * kf;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) rn[i] = __builtin_amdgcn_rsqf(row_sum<16>(ss[i]) + kNormEps);
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int j = 16 * kb + lr;
    const float egn = cp.sEgn[j];
    float gn = 0.f;
    // this lane's four rows of column j: one transposing read per bf16 tile, one read
    // of the key-major e^{G} tile
    const bf16x4 k4 = read_tr4(sK, LDK, 16 * wave + 4 * lq + (lr >> 2), 16 * kb + 4 * (lr & 3));
    const bf16x4 q4 = read_tr4(sQ, LDK, 16 * wave + 4 * lq + (lr >> 2), 16 * kb + 4 * (lr & 3));
    const f32x4 eg4 = *reinterpret_cast<const f32x4*>(cp.sEG + CP::eg_at(j, 16 * wave + 4 * lq));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * lq + i;
      float kf = static_cast<float>(k4[i]);
      if (norm_k) kf = static_cast<float>(static_cast<bf16>(kf * rn[i]));
      const float qf = static_cast<float>(q4[i]);
      const float eg = eg4[i];
      const float ieg = __builtin_amdgcn_rcpf(eg);
      const float eh = egn * ieg;   // e^{G_n - G_r}
      const float dkg = bt[i] * dBk[kb][i];
      const float kg = kf * eg, ki = kf * ieg, kh = kf * eh, qg = a.scale * qf * eg;
      dbk[i] += dBk[kb][i] * kg;
      gn += dKh[kb][i] * kh;
      gm[kb][i] = dkg * kg + dQg[kb][i] * qg - dKi[kb][i] * ki - dKh[kb][i] * kh;
      const float dkv = dkg * eg + dKi[kb][i] * ieg + dKh[kb][i] * eh;
      if (norm_k) {
        dkh[kb][i] = dkv;
        kdot[i] += dkv * kf;
      } else {
        sK[r * LDK + j] = static_cast<bf16>(dkv);
      }
      sQ[r * LDK + j] = static_cast<bf16>(a.scale * dQg[kb][i] * eg);
    }
    // suffix over this lane's four rows, then over the lane groups below it
    gm[kb][2] += gm[kb][3];
    gm[kb][1] += gm[kb][2];
    gm[kb][0] += gm[kb][1];
    const float t = gm[kb][0];
    const float t1 = __shfl(t, (lane + 16) & 63), t2 = __shfl(t, (lane + 32) & 63),
                t3 = __shfl(t, (lane + 48) & 63);
    const float below = (lq < 3 ? t1 : 0.f) + (lq < 2 ? t2 : 0.f) + (lq < 1 ? t3 : 0.f);
    gm[kb] += below;
    gn += __shfl_xor(gn, 16);
    gn += __shfl_xor(gn, 32);
    if (lq == 0) {
      sRed[wave * DK + j] = t + below;          // this token block's column total
      sRed[(4 + wave) * DK + j] = gn;
    }
  }
  // d e^{G_n}: the threads holding the same eight keys (equal tid mod DK / 8) add up,
  // within the wave by shuffles and across the waves in the dg stage
  {
    constexpr int G = DK / 8;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int m = G; m < 64; m *= 2) ddk[e] += __shfl_xor(ddk[e], m);
    if (lane < G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sRed[(8 + wave) * DK + 8 * lane + e] = ddk[e];
    }
  }
  if (norm_k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kdot[i] = row_sum<16>(kdot[i]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16& e = sK[(16 * wave + 4 * lq + i) * LDK + 16 * kb + lr];
        const float kh = static_cast<float>(static_cast<bf16>(static_cast<float>(e) * rn[i]));
        e = static_cast<bf16>((dkh[kb][i] - kh * kdot[i]) * rn[i]);
      }
  }
  // d beta: the V and the Kg terms, summed over this row's values / keys (beta from a
  // logit b: times d sigmoid(b) / db = beta (1 - beta))
  {
    f32x4 tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] = row_sum<16>(dbu[i] + dbk[i]);
    if (a.flags & kBetaLogit) tot *= bt * (1.f - bt);
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * lq + i;
        if (r < n) a.dbeta[(c0 + r) * a.H + h] = tot[i];
      }
    }
  }
  lds_barrier();
  KDA_PHASE(gt_[7] = __builtin_amdgcn_s_memtime();)

  // dq, dk rows
  {
    bf16* dqout = static_cast<bf16*>(a.dq);
    bf16* dkout = static_cast<bf16*>(a.dk);
    for (int i = tid; i < kChunk * DK / 8; i += kThreads) {
      const int r = i / (DK / 8), c8 = 8 * (i % (DK / 8));
      if (r < n) {
        const int64_t off = (c0 + r) * rowK + int64_t(h) * DK + c8;
        *reinterpret_cast<bf16x8*>(dkout + off) = *reinterpret_cast<const bf16x8*>(sK + r * LDK + c8);
        *reinterpret_cast<bf16x8*>(dqout + off) = *reinterpret_cast<const bf16x8*>(sQ + r * LDK + c8);
      }
    }
  }

  // dg: G_r = g_1 + ... + g_r and G_n = G_last, so dg_s = sum_{r >= s} dG_r + dG_n with
  // dG_n = sum_r dKh Kh + d e^{G_n} e^{G_n}.  Per key channel the values go through an
  // LDS tile in area 1 (free once the dq, dk rows have left) and leave as 16-byte pieces.
  float* sDG = reinterpret_cast<float*>(smem + GL::a1);
  constexpr int LDG = GL::LDG;
  if constexpr (DECAY != 2) {
    // What every row of token block w adds to its own suffix sum, once per key column:
    // dG_n (the d e^{G_n} and dKh Kh partials of all waves) plus the column totals of
    // the token blocks after w.  Row w of the reduction scratch takes it (one thread per
    // column reads and writes only that column).
    if (tid < DK) {
      const int j = tid;
      float base = (sRed[8 * DK + j] + sRed[9 * DK + j] + sRed[10 * DK + j] + sRed[11 * DK + j]) *
                   cp.sEgn[j];
      base += sRed[4 * DK + j] + sRed[5 * DK + j] + sRed[6 * DK + j] + sRed[7 * DK + j];
      const float t1 = sRed[DK + j], t2 = sRed[2 * DK + j], t3 = sRed[3 * DK + j];
      sRed[3 * DK + j] = base;
      sRed[2 * DK + j] = base + t3;
      sRed[DK + j] = base + t3 + t2;
      sRed[j] = base + t3 + t2 + t1;
    }
    lds_barrier();
    const bool gate_logit = (a.flags & kGateLogit) != 0;
    f32x4 rows = f32x4{0.f, 0.f, 0.f, 0.f};   // one scalar decay: sums over the channels
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int j = 16 * kb + lr;
      const float add = sRed[wave * DK + j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = gm[kb][i] + add;
        if constexpr (DECAY == 0) {
          sDG[(16 * wave + 4 * lq + i) * LDG + j] = v;
        } else {
          rows[i] += v;
        }
      }
    }
    if constexpr (DECAY == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rows[i] = row_sum<16>(rows[i]);
      if (lr == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * wave + 4 * lq + i;
          if (r < n) {
            const int64_t o = (c0 + r) * a.H + h;
            a.dg[o] = gate_logit ? rows[i] * __builtin_amdgcn_rcpf(1.f + exp_hw(a.g[o])) : rows[i];
          }
        }
      }
    }
    if constexpr (DECAY == 0) {
      lds_barrier();
      for (int i = tid; i < kChunk * DK / 4; i += kThreads) {
        const int r = i / (DK / 4), c4 = 4 * (i % (DK / 4));
        if (r < n) {
          const int64_t o = (c0 + r) * rowK + int64_t(h) * DK + c4;
          f32x4 v = *reinterpret_cast<const f32x4*>(sDG + r * LDG + c4);
          if (gate_logit) {
            // g = log sigmoid(a) from a retention logit a: dg/da = sigmoid(-a)
            const f32x4 ga = *reinterpret_cast<const f32x4*>(a.g + o);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= __builtin_amdgcn_rcpf(1.f + exp_hw(ga[e]));
          }
          *reinterpret_cast<f32x4*>(a.dg + o) = v;
        }
      }
    }
  }
  KDA_PHASE({
    gt_[8] = __builtin_amdgcn_s_memtime();
    if (tid == 0 && blockIdx.x < kGradPhaseItems) {
      unsigned int* w = g_grad_phase + blockIdx.x * kGradPhaseWords;
      for (int i = 1; i < 9; ++i) w[i] = static_cast<unsigned>(gt_[i] - gt_[i - 1]);
      for (int i = 0; i < 4; ++i) w[10 + i] = gs_[i];
      w[15] = 1;
    }
  })
}

// ====================================================================================
// Launch
// ====================================================================================

template <int DK, int DECAY>
static hipError_t launch_tiles_k(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_tiles_kernel<DK, DECAY>), dim3(static_cast<unsigned>(a.slots * a.H)),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward_tiles(int dk, const BwdArgs& a, hipStream_t stream) {
  if (dk == 64) {
    if (a.decay == 1) return launch_tiles_k<64, 1>(a, stream);
    if (a.decay == 2) return launch_tiles_k<64, 2>(a, stream);
    return launch_tiles_k<64, 0>(a, stream);
  }
  if (a.decay == 1) return launch_tiles_k<128, 1>(a, stream);
  if (a.decay == 2) return launch_tiles_k<128, 2>(a, stream);
  return launch_tiles_k<128, 0>(a, stream);
}

template <int DK>
static hipError_t launch_chain_k(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_chain_kernel<DK, kBwdChainBV>), dim3(a.units * a.NV), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_backward_chain(int dk, const BwdArgs& a, hipStream_t stream) {
  return dk == 64 ? launch_chain_k<64>(a, stream) : launch_chain_k<128>(a, stream);
}

template <int DK, int DV>
static hipError_t launch_grads_d(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.slots * a.H)), block(kThreads);
  if (a.decay == 1)
    hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, 1>), grid, block, 0, stream, a);
  else if (a.decay == 2)
    hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, 2>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, 0>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward_grads(int dk, const BwdArgs& a, hipStream_t stream) {
  if (dk == 64) return a.DV == 64 ? launch_grads_d<64, 64>(a, stream) : launch_grads_d<64, 128>(a, stream);
  return a.DV == 64 ? launch_grads_d<128, 64>(a, stream) : launch_grads_d<128, 128>(a, stream);
}

}  // namespace kda

#if defined(KDA_PHASE_STAMPS)
// Timing build only: the gradient kernel's per-item phase rows (see g_grad_phase).
namespace {
__global__ void grad_phase_clear_kernel() {
  for (int i = threadIdx.x; i < kda::kGradPhaseItems * kda::kGradPhaseWords; i += blockDim.x)
    kda::g_grad_phase[i] = 0;
}
}  // namespace
extern "C" int kda_grad_phase_words(void) { return kda::kGradPhaseItems * kda::kGradPhaseWords; }
extern "C" int kda_grad_phase_clear(void) {
  hipLaunchKernelGGL(grad_phase_clear_kernel, dim3(1), dim3(256), 0, 0);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
extern "C" int kda_grad_phase_read(unsigned int* host) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(kda::g_grad_phase),
                             sizeof(unsigned int) * kda::kGradPhaseItems * kda::kGradPhaseWords) ==
                 hipSuccess
             ? 0
             : 1;
}
#endif
