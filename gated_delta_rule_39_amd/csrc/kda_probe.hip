// Peak probes (include/kda_probe.h): an HBM stream and a dense bf16 MFMA loop on
// gfx950.  They measure the machine, not the method; the benchmark divides the KDA
// kernels' algorithmic rates by what these reach.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"
#include "kda_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kStreamBlocks = 4096;   // 16 per CU: enough loads in flight to saturate HBM

// Four independent 16-byte loads in flight per thread, then their stores.
__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, size_t n) {
  const size_t stride = size_t(gridDim.x) * kThreads;
  size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                              size_t n, uint32_t* sink) {
  const size_t stride = size_t(gridDim.x) * kThreads;
  size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Eight independent accumulator chains per wave keep the matrix core issuing back to
// back.  The operands depend on the lane, so nothing is folded at compile time.
__global__ __launch_bounds__(kThreads) void probe_mfma_kernel(float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 1e-3f * (lane + e));
    b[e] = static_cast<__bf16>(1.0f - 1e-3f * (lane - e));
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

int32_t kda_probe_read_sink_words(void) { return kStreamBlocks; }

int kda_probe_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst) return KDA_ERR_NULL_ARG;
  if (bytes < 16 || bytes % 16) return KDA_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kStreamBlocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_probe_hbm_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return KDA_ERR_NULL_ARG;
  if (bytes < 16 || bytes % 16) return KDA_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kStreamBlocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_probe_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, hipStream_t stream) {
  if (!sink) return KDA_ERR_NULL_ARG;
  if (workgroups <= 0 || iters <= 0) return KDA_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(kThreads), 0, stream, sink, iters);
  return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
