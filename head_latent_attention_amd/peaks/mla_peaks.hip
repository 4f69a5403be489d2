// Measured machine peaks: streaming read, streaming copy and a dense bf16 matrix-op loop on
// gfx950.  These kernels are measurement probes for the MLA benchmark, not part of the MLA
// path; each writes a checkable value per thread so that nothing it does is optimised away.
#include <hip/hip_runtime.h>

#include "mla_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void peak_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  size_t i = t;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[t] = acc;
}

__global__ __launch_bounds__(256) void peak_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

__device__ inline bf16x8 splat_bf16(float value) {
  // round to nearest even to bf16 (the value is a small ordinary number)
  uint32_t b = __float_as_uint(value);
  b += 0x7FFFu + ((b >> 16) & 1u);
  const unsigned short h = (unsigned short)(b >> 16);
  const u16x8 u = {h, h, h, h, h, h, h, h};
  return __builtin_bit_cast(bf16x8, u);
}

// Four independent accumulation chains per wave, so consecutive ops never wait on each other.
__global__ void peak_mfma16_kernel(int iters, float value, float* __restrict__ sink) {
  const bf16x8 a = splat_bf16(value);
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void peak_mfma32_kernel(int iters, float value, float* __restrict__ sink) {
  const bf16x8 a = splat_bf16(value);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? 0 : -2; }

}  // namespace

extern "C" {

int mla_peak_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, void* stream) {
  if (!src || !sink || n_wg <= 0 || bytes == 0 || bytes % 16 || !aligned16(src)) return -1;
  hipLaunchKernelGGL(peak_read_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     bytes / 16, sink);
  return launched();
}

int mla_peak_copy(const void* src, void* dst, size_t bytes, int n_wg, void* stream) {
  if (!src || !dst || n_wg <= 0 || bytes == 0 || bytes % 16 || !aligned16(src) || !aligned16(dst)) return -1;
  const char* s = (const char*)src;
  const char* d = (const char*)dst;
  if (s < d + bytes && d < s + bytes) return -1;
  hipLaunchKernelGGL(peak_copy_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     (uint4*)dst, bytes / 16);
  return launched();
}

int mla_peak_mfma_bf16(int shape, int iters, float value, float* sink, int n_wg, int threads, void* stream) {
  if (!sink || n_wg <= 0 || iters <= 0 || (threads != 256 && threads != 512) || (shape != 16 && shape != 32))
    return -1;
  if (shape == 16)
    hipLaunchKernelGGL(peak_mfma16_kernel, dim3(n_wg), dim3(threads), 0, (hipStream_t)stream, iters, value, sink);
  else
    hipLaunchKernelGGL(peak_mfma32_kernel, dim3(n_wg), dim3(threads), 0, (hipStream_t)stream, iters, value, sink);
  return launched();
}

}  // extern "C"
