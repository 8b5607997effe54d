// Host side of the C ABI declared in include/kda.h: argument validation, launch
// geometry and dispatch to the gfx950 kernels.  Validation happens before any HIP
// call, so every status except KDA_ERR_HIP can be produced without a GPU.

#include "kda.h"
#include "kda_noalloc.h"

#include <atomic>
#include <cstdlib>
#include <hip/hip_runtime_api.h>

#include "kda_bwd_launch.h"
#include "kda_launch.h"

namespace {

constexpr int kAllFlags = KDA_PRO_NORM_K | KDA_PRO_BETA_LOGIT | KDA_PRO_GATE_LOGIT;
static_assert(KDA_PRO_NORM_K == kda::kNormK && KDA_PRO_BETA_LOGIT == kda::kBetaLogit &&
                  KDA_PRO_GATE_LOGIT == kda::kGateLogit,
              "prologue flags of the C ABI and the kernels agree");

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not yet queried

// Compute units of the current device (queried once per device, then cached).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = g_cu_count[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

// Value-tile height for the prefill: the smallest number of d_v tiles that gives
// at least one workgroup per compute unit (each workgroup occupies a whole CU's
// LDS), bounded by 16-row tiles and by what the instantiation supports.  The
// environment variable KDA_PREFILL_BV (16, 32, 64) overrides it for tuning.
int choose_bv(int dtype, int32_t units, int32_t dk, int32_t dv, int cus) {
  const int maxbv = kda::prefill_max_bv(dtype, dk) < dv ? kda::prefill_max_bv(dtype, dk) : dv;
  if (const char* e = std::getenv("KDA_PREFILL_BV")) {
    const int b = std::atoi(e);
    if ((b == 16 || b == 32 || b == 64) && b <= maxbv) return b;
  }
  int bv = maxbv;
  while (bv > 16 && static_cast<int64_t>(units) * (dv / bv) < cus) bv /= 2;
  return bv;
}

int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  return e ? std::atoi(e) : dflt;
}

// Producer/consumer geometry: W = CUs / units workgroups per unit (all resident at
// once, one per CU): NC consumers, each 4 waves owning d_v / (4 NC) value columns
// (NC = 2 for d_v = 128 when W >= 6, else 1), and NP = min(W - NC, max_np) producers
// (max_producers: six, or five for a call without decay, whose consumers set the pace
// sooner), and ring_slots(NP) ring slots.  Needs bf16 inputs and W >= 2.  KDA_PREFILL_COOP=0
// disables it; KDA_COOP_NC / KDA_COOP_NP / KDA_COOP_R override the split and the ring
// depth (tuning only).
// Lanes: with d_k = d_v = 128, when the units leave fewer than four workgroups each
// (measured: a unit per set of four still beats two units one after another on seven),
// the units are spread over lanes of seven workgroups (two consumers, five producers;
// as many lanes as the device fits, rounded down to whole XCD groups; a sixth producer
// per lane where the grid has room, as max_producers says) by a plan made
// on the device from cu_seqlens (coop_prep_kernel), longest sequences first, and each
// lane works through its units one after another.  This keeps every unit on the
// producer/consumer kernel however many there are, and balances sequences of unequal
// length.  Up to 256 sequences and 8192 units; KDA_COOP_LANES=0 disables it, =2 takes
// it whenever the units outnumber the lanes (tuning only).
constexpr int kLaneW = 7, kLaneMinW = 4;
// Ring slots per lane.  With five or six producers, 32 (same-box sweeps at T=65536,
// H=32, ms per launch, six producers: R = 12 1.525, 16 1.495, 20 1.456, 24 1.449-1.451,
// 32 1.417, 40 1.411, 48 1.410; B16 H32 T4096 1.441 at 24, 1.403 at 32; varlen 0.658 at
// 24, 0.629 at 32; earlier, five producers: 11 1.650, 24 1.537): the deeper ring lets
// the producers run ahead through the consumers' jitter.  Fewer producers: NP + 6 (B4
// H16 T4096 at NP = 3: 9 and 14 slots measure the same).  Every default plan on a
// 256-CU device stays within 85 MiB of workspace (d_k = 128, d_v = 64, 42 units).
constexpr int kDeepRing = 32;
int ring_slots(int np) { return np >= 5 ? kDeepRing : np + 6; }
constexpr int kPlanMaxSeqs = 256, kPlanMaxUnits = 8192, kPlanMaxLanes = 64;
struct CoopPlan {
  int NC = 0, NP = 0, R = 0, lanes = 0;
  bool plan = false;   // lanes < units: a device plan spreads the units over the lanes
  bool ok() const { return NC > 0; }
};
// Producers per lane for a prefill call.  Six where the producers set the pace — any
// decay, or the prologue flags (then they also normalise keys and turn logits into
// gates) — and five without decay, whose consumers set it (same box, T=65536, H=32:
// per-channel decay 1.435 ms with six against 1.517 with five, per-head decay 1.360 vs
// 1.501, the prologue flags 1.432 vs 1.638, no decay 1.445 vs 1.344; B=16, H=32,
// T=4096 1.477 vs 1.533; the varlen workload 0.662 vs 0.663).  The backward's sweep,
// measured no faster with six, keeps five.
int max_producers(int decay, int flags) { return (flags != 0 || decay != KDA_DECAY_NONE) ? 6 : 5; }
// max_np: producers per lane where the grid has room for them (max_producers below).
// Neither the workspace size nor the lane count depends on it.
CoopPlan coop_plan(int dtype, int64_t units, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                   int cus, int max_np) {
  CoopPlan p;
  if (dtype != KDA_BF16 || units <= 0 || env_int("KDA_PREFILL_COOP", 1) == 0) return p;
  // the producers read a chunk's inputs through buffer resources with 31-bit byte
  // offsets: 64 rows of g (H d_k fp32) and of v (H d_v bf16) must fit
  const int64_t row = static_cast<int64_t>(H) * (d_k * 4 > d_v * 2 ? d_k * 4 : d_v * 2);
  if (64 * row > 0x7fffffff) return p;
  const int enp = env_int("KDA_COOP_NP", 0);
  const int lw = enp > 0 ? 2 + enp : kLaneW;
  int L = cus / lw < kPlanMaxLanes ? cus / lw : kPlanMaxLanes;
  L -= L % 8;
  const int lanes_mode = env_int("KDA_COOP_LANES", 1);   // 0 off, 1 auto, 2 whenever units > L
  if (d_k == 128 && d_v == 128 && (units > cus / kLaneMinW || lanes_mode == 2) && units > L &&
      L >= 8 && N <= kPlanMaxSeqs && units <= kPlanMaxUnits && lanes_mode != 0) {
    p.NC = 2;
    p.NP = lw - 2;
    if (enp == 0 && max_np > kLaneW - 2 && L * (kLaneW + 1) <= cus) p.NP = kLaneW - 1;
    p.R = env_int("KDA_COOP_R", ring_slots(p.NP));
    if (p.R < 3) p.R = 3;
    p.lanes = L;
    p.plan = true;
    return p;
  }
  int W = static_cast<int>(cus / units);
  if (W > 16) W = 16;
  if (W < 2) return p;
  int nc = (d_v == 128 && W >= 6) ? 2 : 1;
  const int enc = env_int("KDA_COOP_NC", 0);
  if (enc > 0 && d_v % (4 * enc) == 0 && (d_v / (4 * enc) == 16 || d_v / (4 * enc) == 32)) nc = enc;
  int np = W - nc < max_np ? W - nc : max_np;
  if (enp > 0) np = enp;
  if (np < 1 || static_cast<int64_t>(units) * (nc + np) > cus) return p;
  p.NC = nc;
  p.NP = np;
  // the split consumer releases chunk c's slot at the start of chunk c + 1, after it
  // has waited for chunk c + 2: three slots at least, or that wait never ends
  p.R = env_int("KDA_COOP_R", ring_slots(np));
  if (p.R < 3) p.R = 3;
  p.lanes = static_cast<int>(units);
  return p;
}

size_t coop_ws_bytes(const CoopPlan& p, int32_t d_k, int32_t d_v, int64_t units) {
  return kda::prefill_coop_workspace_bytes(d_k, d_v, p.lanes, static_cast<int>(units), p.R, p.plan);
}

// The producer/consumer fields of the kernel arguments; the lane plan lives right after
// the workspace header.
void set_coop(kda::PrefillArgs& a, const CoopPlan& p, void* ws) {
  a.workspace = static_cast<unsigned char*>(ws);
  a.NC = p.NC;
  a.NP = p.NP;
  a.R = p.R;
  a.lanes = p.lanes;
  a.xcd_remap = (p.lanes % 8 == 0) ? 1 : 0;
  a.lane_off = p.plan ? reinterpret_cast<const int32_t*>(a.workspace + 256) : nullptr;
  a.lane_units = p.plan ? a.lane_off + p.lanes + 1 : nullptr;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_NULL_ARG: return "KDA_ERR_NULL_ARG: a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: negative or inconsistent sizes";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: d_k and d_v must each be 64 or 128";
    case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE: dtype must be KDA_F32 (0) or KDA_BF16 (1)";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP kernel launch failed";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_SCRATCH:
      return "KDA_ERR_SCRATCH: the call needs more workspace than the allocation-free entry "
             "point's fixed scratch (kda_noalloc_scratch_bytes()); pass a workspace to "
             "kda_prefill_ex instead";
    default: return "KDA: unknown status code";
  }
}

size_t kda_prefill_workspace_bytes(int dtype, int32_t N, int64_t T_total, int32_t H, int32_t d_k,
                                   int32_t d_v) {
  (void)T_total;
  if (N <= 0 || H <= 0 || !supported_dim(d_k) || !supported_dim(d_v)) return 0;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > (1 << 24)) return 0;
  const CoopPlan p = coop_plan(dtype, units, N, H, d_k, d_v, cu_count(),
                               max_producers(KDA_DECAY_CHANNEL, 0));
  if (!p.ok()) return 0;
  return coop_ws_bytes(p, d_k, d_v, units);
}

int kda_prefill_coop_plan(int dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                          int32_t* consumers, int32_t* producers, int32_t* ring_slots) {
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (N < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > (1 << 24)) return KDA_ERR_BAD_SHAPE;
  const CoopPlan p = coop_plan(dtype, units, N, H, d_k, d_v, cu_count(),
                               max_producers(KDA_DECAY_CHANNEL, 0));
  if (consumers) *consumers = p.NC;
  if (producers) *producers = p.NP;
  if (ring_slots) *ring_slots = p.R;
  return KDA_OK;
}

int kda_prefill_coop_lanes(int dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v) {
  if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
  if (N <= 0 || H <= 0 || !supported_dim(d_k) || !supported_dim(d_v)) return 0;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > (1 << 24)) return 0;
  const CoopPlan p = coop_plan(dtype, units, N, H, d_k, d_v, cu_count(),
                               max_producers(KDA_DECAY_CHANNEL, 0));
  return p.ok() ? p.lanes : 0;
}

int kda_prefill_plan(int dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                     int32_t* v_tiles, int32_t* workgroups) {
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (N < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > (1 << 24)) return KDA_ERR_BAD_SHAPE;
  const int bv = choose_bv(dtype, static_cast<int32_t>(units), d_k, d_v, cu_count());
  if (v_tiles) *v_tiles = d_v / bv;
  if (workgroups) *workgroups = static_cast<int32_t>(units * (d_v / bv));
  return KDA_OK;
}

}  // extern "C"

namespace kda {
// Argument checks of kda_prefill_ex (no HIP call).  KDA_OK with *launch = false when
// there is nothing to do.
int prefill_args_status(int dtype, int decay, int flags, const void* q, const void* k,
                        const void* v, const float* g, const float* beta,
                        const int32_t* cu_seqlens, int32_t N, int32_t B, int64_t T, int32_t H,
                        int32_t d_k, int32_t d_v, const float* final_state, const void* o,
                        bool* launch) {
  *launch = false;
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (decay != KDA_DECAY_CHANNEL && decay != KDA_DECAY_HEAD && decay != KDA_DECAY_NONE)
    return KDA_ERR_UNSUPPORTED;
  if (flags & ~kAllFlags) return KDA_ERR_UNSUPPORTED;
  if (N < 0 || B < 0 || T < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens == nullptr && N != B) return KDA_ERR_BAD_SHAPE;
  if (cu_seqlens != nullptr && B != 1) return KDA_ERR_BAD_SHAPE;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > (1 << 24)) return KDA_ERR_BAD_SHAPE;
  if (N == 0) return KDA_OK;
  // with every sequence empty only the state copy remains; it is still launched.
  if (static_cast<int64_t>(B) * T > 0 &&
      (!q || !k || !v || (!g && decay != KDA_DECAY_NONE) || !beta || !o))
    return KDA_ERR_NULL_ARG;
  if (static_cast<int64_t>(B) * T == 0 && !final_state) return KDA_OK;
  *launch = true;
  return KDA_OK;
}
}  // namespace kda

extern "C" {

int kda_prefill_ex(int dtype, int decay, int flags, const void* q, const void* k,
                   const void* v, const float* g, const float* beta, const int32_t* cu_seqlens,
                   int32_t N, int32_t B, int64_t T, int32_t H, int32_t d_k, int32_t d_v,
                   float scale, const float* initial_state, float* final_state, void* o,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool launch = false;
  const int st = kda::prefill_args_status(dtype, decay, flags, q, k, v, g, beta, cu_seqlens, N, B,
                                          T, H, d_k, d_v, final_state, o, &launch);
  if (st != KDA_OK || !launch) return st;
  const int64_t units = static_cast<int64_t>(N) * H;
  kda::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu_seqlens = cu_seqlens;
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.o = o;
  a.T = T;
  a.H = H;
  a.DV = d_v;
  a.units = static_cast<int32_t>(units);
  a.xcd_remap = (units % 8 == 0) ? 1 : 0;
  a.scale = scale;
  a.decay = decay;
  a.flags = flags;
  const int cus = cu_count();
  const CoopPlan p = coop_plan(dtype, units, N, H, d_k, d_v, cus, max_producers(decay, flags));
  if (p.ok() && workspace != nullptr && workspace_bytes >= coop_ws_bytes(p, d_k, d_v, units)) {
    set_coop(a, p, workspace);
    if (kda::launch_prefill_coop(d_k, a, stream) == hipSuccess) return KDA_OK;
    (void)hipGetLastError();   // not launchable as one resident grid: use the fused kernel
    a.xcd_remap = (units % 8 == 0) ? 1 : 0;
    a.lane_off = a.lane_units = nullptr;
  }
  const int bv = choose_bv(dtype, static_cast<int32_t>(units), d_k, d_v, cus);
  a.NV = d_v / bv;
  a.workspace = nullptr;
  hipError_t err = kda::launch_prefill(dtype, d_k, bv, a, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_prefill(int dtype, const void* q, const void* k, const void* v, const float* g,
                const float* beta, const int32_t* cu_seqlens, int32_t N, int32_t B, int64_t T,
                int32_t H, int32_t d_k, int32_t d_v, float scale, const float* initial_state,
                float* final_state, void* o, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return kda_prefill_ex(dtype, KDA_DECAY_CHANNEL, 0, q, k, v, g, beta, cu_seqlens, N, B, T, H, d_k,
                        d_v, scale, initial_state, final_state, o, workspace, workspace_bytes,
                        stream);
}

int kda_decode_step_ex(int dtype, int decay, int flags, const void* q, const void* k,
                       const void* v, const float* g, const float* beta, float* state, void* o,
                       int32_t N, int32_t H, int32_t d_k, int32_t d_v, float scale,
                       hipStream_t stream) {
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (decay != KDA_DECAY_CHANNEL && decay != KDA_DECAY_HEAD && decay != KDA_DECAY_NONE)
    return KDA_ERR_UNSUPPORTED;
  if (flags & ~kAllFlags) return KDA_ERR_UNSUPPORTED;
  if (N < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > 0x7fffffff) return KDA_ERR_BAD_SHAPE;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || (!g && decay != KDA_DECAY_NONE) || !beta || !state || !o)
    return KDA_ERR_NULL_ARG;
  hipError_t err = kda::launch_decode(dtype, decay, flags, d_k, d_v, q, k, v, g, beta, state, o,
                                      static_cast<int32_t>(units), scale, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step(int dtype, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, float* state, void* o, int32_t N, int32_t H,
                    int32_t d_k, int32_t d_v, float scale, hipStream_t stream) {
  return kda_decode_step_ex(dtype, KDA_DECAY_CHANNEL, 0, q, k, v, g, beta, state, o, N, H, d_k,
                            d_v, scale, stream);
}

}  // extern "C"

namespace {
// Backward workspace: [producer/consumer ring of the forward sweep, when that kernel
// applies (d_k = d_v = 128, two consumers) | chunk states | state gradients | chunk
// tiles of the reverse chain].
struct BwdPlan {
  CoopPlan coop;
  size_t ring = 0, states = 0, tiles = 0;
  size_t total() const { return ring + 2 * states + tiles; }
};
BwdPlan bwd_plan(int32_t N, int64_t T_total, int32_t H, int32_t d_k, int32_t d_v) {
  BwdPlan b;
  const int64_t units = static_cast<int64_t>(N) * H;
  b.states = static_cast<size_t>(kda::chunk_slots_host(T_total, N) * H * d_v * d_k * 2);
  b.tiles = static_cast<size_t>(kda::chunk_slots_host(T_total, N) * H) * kda::chain_tile_bytes(d_k);
  CoopPlan p = coop_plan(KDA_BF16, units, N, H, d_k, d_v, cu_count(), 5);
  // the sweep keeps NP + 6 slots: the deeper forward ring measured no faster here
  // (8.33-8.39 vs 8.40-8.42 ms per call at T=65536, H=32) and costs 30 MB more
  if (p.ok()) p.R = env_int("KDA_COOP_R", p.NP + 6);
  if (p.ok() && d_k == 128 && d_v == 128 && p.NC == 2 && units <= (1 << 24)) {
    b.coop = p;
    b.ring = (coop_ws_bytes(p, d_k, d_v, units) + 255) & ~size_t(255);
  }
  return b;
}
}  // namespace

extern "C" {

size_t kda_backward_workspace_bytes(int dtype, int32_t N, int64_t T_total, int32_t H, int32_t d_k,
                                    int32_t d_v) {
  if (dtype != KDA_BF16 || N <= 0 || T_total < 0 || H <= 0 || !supported_dim(d_k) ||
      !supported_dim(d_v))
    return 0;
  return bwd_plan(N, T_total, H, d_k, d_v).total();
}

int kda_backward(int dtype, int decay, int flags, const void* q, const void* k, const void* v,
                 const float* g, const float* beta, const int32_t* cu_seqlens, int32_t N,
                 int32_t B, int64_t T, int32_t H, int32_t d_k, int32_t d_v, float scale,
                 const float* initial_state, const void* dout, const float* dfinal_state,
                 void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dinitial_state,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (decay != KDA_DECAY_CHANNEL && decay != KDA_DECAY_HEAD && decay != KDA_DECAY_NONE)
    return KDA_ERR_UNSUPPORTED;
  if (flags & ~kAllFlags) return KDA_ERR_UNSUPPORTED;
  if (N < 0 || B < 0 || T < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens == nullptr && N != B) return KDA_ERR_BAD_SHAPE;
  if (cu_seqlens != nullptr && B != 1) return KDA_ERR_BAD_SHAPE;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > (1 << 24)) return KDA_ERR_BAD_SHAPE;
  if (N == 0) return KDA_OK;
  const int64_t tot = static_cast<int64_t>(B) * T;
  const int64_t slots = kda::chunk_slots_host(tot, N);
  if (slots * H > 0x7fffffff) return KDA_ERR_BAD_SHAPE;
  if (tot > 0 && (!q || !k || !v || (decay != KDA_DECAY_NONE && (!g || !dg)) || !beta || !dout ||
                  !dq || !dk || !dv || !dbeta))
    return KDA_ERR_NULL_ARG;
  const BwdPlan plan = bwd_plan(N, tot, H, d_k, d_v);
  if (workspace == nullptr || workspace_bytes < plan.total()) return KDA_ERR_WORKSPACE;
  if (tot == 0 && !dinitial_state) return KDA_OK;
  unsigned char* states = static_cast<unsigned char*>(workspace) + plan.ring;
  unsigned char* dstates = states + plan.states;
  const int cus = cu_count();
  bool tiles_done = false;   // the producer/consumer sweep also wrote the chunk tiles
  if (tot > 0) {
    kda::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.initial_state = initial_state;
    a.T = T;
    a.H = H;
    a.DV = d_v;
    a.units = static_cast<int32_t>(units);
    a.xcd_remap = (units % 8 == 0) ? 1 : 0;
    a.scale = scale;
    a.decay = decay;
    a.flags = flags;
    a.chunk_states = states;
    a.chunk_tiles = dstates + plan.states;
    bool done = false;
    if (plan.ring > 0) {
      set_coop(a, plan.coop, workspace);
      done = kda::launch_prefill_coop_states(a, stream) == hipSuccess;
      if (!done) {
        (void)hipGetLastError();   // not launchable as one resident grid
        a.xcd_remap = (units % 8 == 0) ? 1 : 0;
        a.lane_off = a.lane_units = nullptr;
      }
    }
    tiles_done = done;
    if (!done) {
      a.workspace = nullptr;
      const int bv = choose_bv(KDA_BF16, static_cast<int32_t>(units), d_k, d_v, cus);
      a.NV = d_v / bv;
      if (kda::launch_prefill_states(d_k, bv, a, stream) != hipSuccess) return KDA_ERR_HIP;
    }
  }
  kda::BwdArgs b{};
  b.q = q;
  b.k = k;
  b.v = v;
  b.g = g;
  b.beta = beta;
  b.dout = dout;
  b.cu_seqlens = cu_seqlens;
  b.dfinal_state = dfinal_state;
  b.dinitial_state = dinitial_state;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dg = dg;
  b.dbeta = dbeta;
  b.states = states;
  b.dstates = dstates;
  b.tiles = dstates + plan.states;
  b.T = T;
  b.slots = slots;
  b.H = H;
  b.DV = d_v;
  b.N = N;
  b.units = static_cast<int32_t>(units);
  b.NV = d_v / kda::kBwdChainBV;
  b.xcd_remap = (units % 8 == 0) ? 1 : 0;
  b.decay = decay;
  b.flags = flags;
  b.scale = scale;
  if (tot > 0 && !tiles_done && kda::launch_backward_tiles(d_k, b, stream) != hipSuccess)
    return KDA_ERR_HIP;
  if (kda::launch_backward_chain(d_k, b, stream) != hipSuccess) return KDA_ERR_HIP;
  if (tot > 0 && kda::launch_backward_grads(d_k, b, stream) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"
