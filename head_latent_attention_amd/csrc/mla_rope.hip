// Rotary tables and the layer-input RMSNorm: small HBM-bound row kernels in front of
// the stage-1 projection.
//
//   rope_inv_freq_kernel   per-pair inverse frequencies, plain or YaRN (atlas docs,
//                          Struct MlaWeights, fields yarn_inv_freq / main_inv_freq),
//                          evaluated in fp64
//   rope_tables_kernel     cos/sin [n, dr/2] of angle = position * inv_freq[i]: angle and
//                          its reduction to a quadrant in fp64, cos/sin of the reduced
//                          angle in fp32 (AWS Neuron NKI, "MLA Decode QKV Kernel API
//                          Reference", cos/sin parameters)
//   input_norm_kernel      x * rsqrt(mean(x^2) + eps) * gamma per row (same reference,
//                          input_norm_w parameter), one workgroup per row
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "mla_kernels.h"

namespace mla {
namespace {

// YaRN by parts (Peng et al., "YaRN: Efficient Context Window Extension of Large Language
// Models", section 3.2): a pair whose wavelength turns at least beta_fast times over the
// original context keeps its frequency, one that turns at most beta_slow times is divided
// by the factor, and the share of the divided frequency grows linearly in the pair index
// between the two (bounds rounded outward).
__global__ void rope_inv_freq_kernel(int dr, double theta, double factor, double L, double beta_fast,
                                     double beta_slow, double* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= dr / 2) return;
  const double plain = pow(theta, -2.0 * i / dr);
  if (!(factor > 1.0)) {
    out[i] = plain;
    return;
  }
  const double two_pi = 6.283185307179586476925286766559;
  // pair index at which the wavelength turns n times over L positions
  const double at_fast = dr * log(L / (beta_fast * two_pi)) / (2.0 * log(theta));
  const double at_slow = dr * log(L / (beta_slow * two_pi)) / (2.0 * log(theta));
  const double lo = fmax(floor(at_fast), 0.0);
  const double hi = fmin(ceil(at_slow), (double)(dr - 1));
  double share;  // share of the divided frequency
  if (hi > lo)
    share = fmin(fmax((i - lo) / (hi - lo), 0.0), 1.0);
  else
    share = i > lo ? 1.0 : 0.0;
  out[i] = plain / factor * share + plain * (1.0 - share);
}

// IDX: the index type of the flattened [n, half] table (32-bit division where the table allows).
template <typename IDX>
__global__ void rope_tables_kernel(IDX total, int half, const int32_t* __restrict__ positions, int pos_offset,
                                   const double* __restrict__ inv_freq, float* __restrict__ cosT,
                                   float* __restrict__ sinT) {
  for (IDX e = blockIdx.x * (IDX)blockDim.x + threadIdx.x; e < total; e += (IDX)gridDim.x * blockDim.x) {
    const IDX t = e / (IDX)half;
    const int i = (int)(e - t * (IDX)half);
    const int64_t pos = (int64_t)(positions ? positions[t] : (int64_t)t) + pos_offset;
    const double f = inv_freq ? inv_freq[i] : pow(10000.0, -2.0 * i / (2 * half));
    // the angle and its reduction to a quadrant, a = q pi/2 + r with |r| <= pi/4 (up to the
    // rounding of a * 2/pi near a quadrant boundary), in fp64: r is one fused multiply-add,
    // exact to ~1e-11 rad up to 1e5 rad; then fp32 cos/sin of r (rounding r to fp32 costs
    // <= 3e-8 rad) rotated by the quadrant: a few fp32 ulps, at a fraction of fp64 sincos's cost
    const double a = (double)pos * f;
    const double half_pi = 1.5707963267948966192313216916398;
    const double two_over_pi = 0.63661977236758134307553505349006;
    const double qd = rint(a * two_over_pi);
    float sr, cr;
    sincosf((float)fma(-qd, half_pi, a), &sr, &cr);
    const int quad = (int)((int64_t)qd & 3);
    const float c = quad == 0 ? cr : quad == 1 ? -sr : quad == 2 ? -cr : sr;
    const float sn = quad == 0 ? sr : quad == 1 ? cr : quad == 2 ? -sr : -cr;
    cosT[e] = c;
    sinT[e] = sn;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void input_norm_kernel(const T* __restrict__ x, int D, const float* __restrict__ g,
                                                         float eps, T* __restrict__ y) {
  __shared__ float red[16];
  const T* xr = x + (int64_t)blockIdx.x * D;
  T* yr = y + (int64_t)blockIdx.x * D;
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    const float v = Act<T>::ld(xr, i);
    ss += v * v;
  }
  const float r = rsqrtf(block_sum(ss, red) / (float)D + eps);
  for (int i = threadIdx.x; i < D; i += blockDim.x) Act<T>::st(yr, i, Act<T>::ld(xr, i) * r * g[i]);
}

// bf16 rows with D % 8 == 0: 16-byte loads and stores, the row held in registers between
// the two passes when it fits (D <= 256 * 8 * kVec).
constexpr int kVec = 4;
__global__ __launch_bounds__(256) void input_norm_bf16x8_kernel(const bf16_t* __restrict__ x, int D,
                                                                const float* __restrict__ g, float eps,
                                                                bf16_t* __restrict__ y) {
  __shared__ float red[16];
  const int chunks = D / 8;
  const uint4* xr = (const uint4*)(x + (int64_t)blockIdx.x * D);
  uint4* yr = (uint4*)(y + (int64_t)blockIdx.x * D);
  uint4 v[kVec];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int c = threadIdx.x + j * 256;
    v[j] = c < chunks ? xr[c] : make_uint4(0, 0, 0, 0);
  }
  for (int c = threadIdx.x + kVec * 256; c < chunks; c += 256) {  // rows beyond the register cache
    const uint4 u = xr[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_to_f32((uint16_t)(w[e] & 0xFFFF)), b = bf16_to_f32((uint16_t)(w[e] >> 16));
      ss += a * a + b * b;
    }
  }
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_to_f32((uint16_t)(w[e] & 0xFFFF)), b = bf16_to_f32((uint16_t)(w[e] >> 16));
      ss += a * a + b * b;
    }
  }
  const float r = rsqrtf(block_sum(ss, red) / (float)D + eps);
  auto emit = [&](int c, const uint4& u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const float4 g0 = ((const float4*)g)[2 * c], g1 = ((const float4*)g)[2 * c + 1];
    const float gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = bf16_to_f32((uint16_t)(w[e] & 0xFFFF)), b = bf16_to_f32((uint16_t)(w[e] >> 16));
      o[e] = pack_bf16x2(a * r * gs[2 * e], b * r * gs[2 * e + 1]);
    }
    yr[c] = make_uint4(o[0], o[1], o[2], o[3]);
  };
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c < chunks) emit(c, v[j]);
  }
  for (int c = threadIdx.x + kVec * 256; c < chunks; c += 256) emit(c, xr[c]);
}

}  // namespace

hipError_t rope_inv_freq(int dr, double theta, double factor, int original_max_position, double beta_fast,
                         double beta_slow, double* inv_freq, hipStream_t s) {
  const int half = dr / 2;
  rope_inv_freq_kernel<<<(half + 63) / 64, 64, 0, s>>>(dr, theta, factor, (double)original_max_position, beta_fast,
                                                       beta_slow, inv_freq);
  return hipGetLastError();
}

hipError_t rope_tables(int n, int dr, const int32_t* positions, int pos_offset, const double* inv_freq, float* cosT,
                       float* sinT, hipStream_t s) {
  const int half = dr / 2;
  const int64_t total = (int64_t)n * half;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  if (total <= INT32_MAX)
    rope_tables_kernel<uint32_t><<<blocks, 256, 0, s>>>((uint32_t)total, half, positions, pos_offset, inv_freq, cosT,
                                                        sinT);
  else
    rope_tables_kernel<int64_t><<<blocks, 256, 0, s>>>(total, half, positions, pos_offset, inv_freq, cosT, sinT);
  return hipGetLastError();
}

hipError_t input_norm(const Dims& d, const void* x, int n, const float* gamma, void* y, hipStream_t s) {
  if (d.act == 1 && d.D % 8 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)gamma & 15) == 0)
    input_norm_bf16x8_kernel<<<n, 256, 0, s>>>((const bf16_t*)x, d.D, gamma, d.eps, (bf16_t*)y);
  else if (d.act == 1)
    input_norm_kernel<bf16_t><<<n, 256, 0, s>>>((const bf16_t*)x, d.D, gamma, d.eps, (bf16_t*)y);
  else
    input_norm_kernel<float><<<n, 256, 0, s>>>((const float*)x, d.D, gamma, d.eps, (float*)y);
  return hipGetLastError();
}

}  // namespace mla
