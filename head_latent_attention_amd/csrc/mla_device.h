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
  // gfx950 v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats to a packed pair of bf16 (a in the low half), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
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

// Reductions over the lanes that share (lane & 15): the gfx950 row-swap permutes
// (v_permlane16_swap / v_permlane32_swap) leave {x[l], x[l ^ 16]} (resp. 32) in the
// two results of every lane.
__device__ __forceinline__ float xmax16_32(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float xsum16_32(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Workgroup barrier without the memory fence of __syncthreads(), which would wait for every
// global->LDS copy still in flight (the prefetched tiles too).  Callers make LDS data safe
// themselves: each wave waits for its own copies of the tile about to be read (vmcnt) and has
// consumed its earlier LDS reads (lgkmcnt) before arriving.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS copy, 16 bytes per lane, through a raw buffer resource based at the
// wave-uniform address `base`: lane l's bytes [base + voff, base + voff + 16) land at
// lds_base + 16*l.  The buffer form (unlike global_load_lds, which the compiler must treat
// as possibly touching the LDS counter) leaves LDS reads issued while copies are in flight
// waitable one by one.  Resource word 3 selects 32-bit data format, as untyped gfx9
// buffer accesses need; every offset used stays below `bytes`.
__device__ __forceinline__ void dma16_buf(const void* base, uint32_t bytes, uint32_t voff, void* lds_base) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}

}  // namespace mla
