// MX fp8 quantisation of activation rows (AWS Neuron NKI, "QKV CTE MLA Kernel API
// Reference": the context-encoding projections run on MX fp8 with 8-bit power-of-two scales).
// Per row and per group of 128 columns: e = the smallest integer with max|x| <= 448 * 2^e
// (0 for an all-zero group, clamped to E8M0's [-127, 127]), codes = E4M3FN(x * 2^-e) rounded
// to nearest even by the hardware conversion.  x * 2^-e is exact, so the code is a function of
// the bf16 input alone.
//
// 16 lanes own one group (8 columns each, a 16-byte load when the row allows it); the group
// maximum is a 4-step lane exchange.  Outputs: codes [M, K] plus E8M0 exponent bytes, or the
// dequantised values code * 2^e as bf16 (exact: 3 mantissa bits), for consumers that take bf16.
#include <hip/hip_runtime.h>

#include "mla_fast.h"
#include "mla_kernels.h"

namespace mla {
namespace {

__global__ __launch_bounds__(256) void quant_mx_kernel(const bf16_t* __restrict__ x, int64_t ldx, int M, int K,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ exps,
                                                       int exp_order, bf16_t* __restrict__ deq) {
  const int G = (K + 127) / 128;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t grp = t >> 4;
  const int sub = (int)(t & 15);
  const bool live = grp < (int64_t)M * G;  // every lane runs the exchange below
  const int m = live ? (int)(grp / G) : 0, gi = live ? (int)(grp - (int64_t)m * G) : 0;
  const int c0 = gi * 128 + sub * 8;
  const bf16_t* row = x + (int64_t)m * ldx;
  float v[8];
  const bool vec = live && c0 + 8 <= K && ((ldx & 7) == 0) && (((uintptr_t)x & 15) == 0);
  if (vec) {
    const uint4 u = *(const uint4*)(row + c0);
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(wv[i] & 0xFFFF));
      v[2 * i + 1] = bf16_to_f32((uint16_t)(wv[i] >> 16));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (live && c0 + i < K) ? bf16_to_f32(row[c0 + i]) : 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  int e = 0;
  if (amax > 0.f) {
    int ex;
    const float mant = frexpf(amax, &ex);  // amax = mant * 2^ex, mant in [0.5, 1); 448 = 0.875 * 2^9
    e = ex - 9 + (mant > 0.875f ? 1 : 0);
    e = max(-127, min(127, e));
  }
  if (!live) return;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = ldexpf(v[i], -e);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  if (deq) {
    bf16_t* drow = deq + (int64_t)m * K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint8_t c = (uint8_t)((uint32_t)(i < 4 ? lo : hi) >> (8 * (i & 3)));
      if (c0 + i < K) drow[c0 + i] = f32_to_bf16(ldexpf(fp8_to_f32(c), e));
    }
  } else {
    uint8_t* crow = codes + (int64_t)m * K;
    if (c0 + 8 <= K && (K & 7) == 0) {
      *(uint2*)(crow + c0) = make_uint2((uint32_t)lo, (uint32_t)hi);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c0 + i < K) crow[c0 + i] = (uint8_t)((uint32_t)(i < 4 ? lo : hi) >> (8 * (i & 3)));
    }
    if (sub == 0) {
      const int64_t m_pad = f8_rows_pad(M);
      exps[exp_order ? f8_exp_order(gi, m, m_pad) : (int64_t)gi * M + m] = (uint8_t)(e + 127);
    }
  }
}

}  // namespace

hipError_t quant_mx(const bf16_t* x, int64_t ldx, int M, int K, uint8_t* codes, uint8_t* exps, bool exp_order,
                    bf16_t* deq, hipStream_t s) {
  if (M <= 0 || K <= 0) return hipSuccess;
  const int64_t threads = (int64_t)M * ((K + 127) / 128) * 16;
  quant_mx_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(x, ldx, M, K, codes, exps, exp_order ? 1 : 0, deq);
  return hipGetLastError();
}

}  // namespace mla
