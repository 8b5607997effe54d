// Host side of the C ABI declared in include/kda.h: argument validation, launch
// geometry and dispatch to the gfx950 kernels.  Validation happens before any HIP
// call, so every status except KDA_ERR_HIP can be produced without a GPU.

#include "kda.h"

#include <atomic>
#include <cstdlib>
#include <hip/hip_runtime_api.h>

namespace kda {
hipError_t launch_decode(int dtype, int dk, int dv, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float* state, void* o,
                         int32_t units, float scale, hipStream_t stream);
hipError_t launch_prefill(int dtype, int dk, int bv, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, const int32_t* cu,
                          int64_t T, int32_t H, int32_t DV, int32_t NV, int32_t units,
                          int32_t xcd_remap, float scale, const float* s0, float* s1, void* o,
                          hipStream_t stream);
int prefill_max_bv(int dtype, int dk);
}  // namespace kda

namespace {

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
    default: return "KDA: unknown status code";
  }
}

size_t kda_prefill_workspace_bytes(int, int32_t, int64_t, int32_t, int32_t, int32_t) { return 0; }

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

int kda_prefill(int dtype, const void* q, const void* k, const void* v, const float* g,
                const float* beta, const int32_t* cu_seqlens, int32_t N, int32_t B, int64_t T,
                int32_t H, int32_t d_k, int32_t d_v, float scale, const float* initial_state,
                float* final_state, void* o, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (N < 0 || B < 0 || T < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens == nullptr && N != B) return KDA_ERR_BAD_SHAPE;
  if (cu_seqlens != nullptr && B != 1) return KDA_ERR_BAD_SHAPE;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > (1 << 24)) return KDA_ERR_BAD_SHAPE;
  if (N == 0) return KDA_OK;
  // with every sequence empty only the state copy remains; it is still launched.
  if (static_cast<int64_t>(B) * T > 0 && (!q || !k || !v || !g || !beta || !o))
    return KDA_ERR_NULL_ARG;
  if (static_cast<int64_t>(B) * T == 0 && !final_state) return KDA_OK;
  const int bv = choose_bv(dtype, static_cast<int32_t>(units), d_k, d_v, cu_count());
  const int32_t nv = d_v / bv;
  const int32_t xcd_remap = (units % 8 == 0) ? 1 : 0;
  hipError_t err = kda::launch_prefill(dtype, d_k, bv, q, k, v, g, beta, cu_seqlens, T, H, d_v,
                                       nv, static_cast<int32_t>(units), xcd_remap, scale,
                                       initial_state, final_state, o, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step(int dtype, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, float* state, void* o, int32_t N, int32_t H,
                    int32_t d_k, int32_t d_v, float scale, hipStream_t stream) {
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (N < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  if (!supported_dim(d_k) || !supported_dim(d_v)) return KDA_ERR_UNSUPPORTED;
  const int64_t units = static_cast<int64_t>(N) * H;
  if (units > 0x7fffffff) return KDA_ERR_BAD_SHAPE;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL_ARG;
  hipError_t err = kda::launch_decode(dtype, d_k, d_v, q, k, v, g, beta, state, o,
                                      static_cast<int32_t>(units), scale, stream);
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
