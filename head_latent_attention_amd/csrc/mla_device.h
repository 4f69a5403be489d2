// Device-side helpers shared by the gfx950 MLA kernels: storage-format
// conversions (fp32, bf16 bit patterns, OCP E4M3FN bytes), wave64 reductions and
// the weight element loader used by the general kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef uint16_t bf16_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One OCP E4M3FN byte to fp32 with the gfx950 conversion instruction.
__device__ __forceinline__ float fp8_to_f32(uint8_t c) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false)[0];
}

// Activation element access: T is float (MLA_F32) or bf16_t (MLA_BF16).
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};
template <> struct Act<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  static __device__ __forceinline__ float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

enum WeightKind { W_F32 = 0, W_BF16 = 1, W_FP8 = 2 };

// A [K, N] row-major weight; for W_FP8 `scale` is fp32 [ceil(K/128), ceil(N/128)].
struct WeightView {
  const void* w;
  const float* scale;
  int64_t ld;        // elements between consecutive k rows
  int scale_ld;      // ceil(N_total/128) of the full matrix
};

template <int WK>
__device__ __forceinline__ float load_w(const WeightView& v, int64_t k, int64_t n) {
  if constexpr (WK == W_F32) {
    return ((const float*)v.w)[k * v.ld + n];
  } else if constexpr (WK == W_BF16) {
    return bf16_to_f32(((const bf16_t*)v.w)[k * v.ld + n]);
  } else {
    float s = v.scale[(k >> 7) * v.scale_ld + (n >> 7)];
    return fp8_to_f32(((const uint8_t*)v.w)[k * v.ld + n]) * s;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024); `red` holds >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

}  // namespace mla
