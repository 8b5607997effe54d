// kda_prefill_noalloc (include/kda_noalloc.h): kda_prefill_ex with the producer/consumer
// kernel's workspace taken from a library-owned device array instead of the caller,
// for callers that cannot allocate.
//
// The array is a file-scope __device__ object: every device the library runs on holds
// its own copy, at its own address, from code-object load until the process ends.  In
// host code its name is only a host-side stand-in, so the device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only that
// address is ever passed on.  The kernels clear what must start at zero (the abort
// word and the hand-off flags) with a fill kernel at every launch; the ring slots are
// always written before they are read.  Calls that overlap on one device race on the
// array.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kda_noalloc.h"
#include "kda_launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch` (nullptr on failure).
void* scratch_ptr(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace

extern "C" {

size_t kda_noalloc_scratch_bytes(void) { return KDA_NOALLOC_SCRATCH_BYTES; }

int kda_prefill_noalloc(int dtype, int decay, int flags, const void* q, const void* k,
                        const void* v, const float* g, const float* beta,
                        const int32_t* cu_seqlens, int32_t N, int32_t B, int64_t T, int32_t H,
                        int32_t d_k, int32_t d_v, float scale, const float* initial_state,
                        float* final_state, void* o, hipStream_t stream) {
  // the argument checks of kda_prefill_ex, before any HIP call
  bool launch = false;
  const int st = kda::prefill_args_status(dtype, decay, flags, q, k, v, g, beta, cu_seqlens, N, B,
                                          T, H, d_k, d_v, final_state, o, &launch);
  if (st != KDA_OK || !launch) return st;
  const size_t need = kda_prefill_workspace_bytes(dtype, N, int64_t(B) * T, H, d_k, d_v);
  if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
  if (need == 0)   // the fused kernel applies: it uses no scratch
    return kda_prefill_ex(dtype, decay, flags, q, k, v, g, beta, cu_seqlens, N, B, T, H, d_k,
                          d_v, scale, initial_state, final_state, o, nullptr, 0, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return KDA_ERR_HIP;
  return kda_prefill_ex(dtype, decay, flags, q, k, v, g, beta, cu_seqlens, N, B, T, H, d_k, d_v,
                        scale, initial_state, final_state, o, ws, KDA_NOALLOC_SCRATCH_BYTES,
                        stream);
}

}  // extern "C"
