// Host-side launchers of the gfx950 MLA kernels.  Every launcher only enqueues
// on `s` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"

namespace mla {

struct Dims {
  int D, H, Lq, Lkv, dn, dr, dv;
  float scale, eps;
  int bs;
  int act;      // 0 f32, 1 bf16
  int wk;       // WeightKind
  int aq = 0;   // 1: activations entering the projections are MX fp8-quantised
  int dqk() const { return dn + dr; }
  int R() const { return Lkv + dr; }
};

// fp32 matrix given as a sum of split-K partial products:
//   value(m, n) = sum_{z < splits} p[z * stride + m * ld + n]
struct Partials {
  const float* p;
  int splits;
  int64_t stride;
  int64_t ld;
  Partials offset(int64_t cols) const { return Partials{p + cols, splits, stride, ld}; }
};

// Sum in a fixed order: four independent running sums (parts z = 0, 1, 2, 3 mod 4) so that
// the loads of a round are in flight together, then (s0 + s1) + (s2 + s3).
__device__ __forceinline__ float part_ld(const Partials& P, int64_t m, int64_t n) {
  const float* q = P.p + m * P.ld + n;
  if (P.splits == 1) return q[0];
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int z = 0;
  for (; z + 4 <= P.splits; z += 4) {
    s0 += q[(int64_t)z * P.stride];
    s1 += q[(int64_t)(z + 1) * P.stride];
    s2 += q[(int64_t)(z + 2) * P.stride];
    s3 += q[(int64_t)(z + 3) * P.stride];
  }
  if (z < P.splits) s0 += q[(int64_t)z * P.stride];
  if (z + 1 < P.splits) s1 += q[(int64_t)(z + 1) * P.stride];
  if (z + 2 < P.splits) s2 += q[(int64_t)(z + 2) * P.stride];
  return (s0 + s1) + (s2 + s3);
}

// part_ld of eight consecutive columns n .. n+7 with 16-byte loads, the same summation order
// (P.p + m * P.ld + n and P.stride keep 16-byte alignment).
__device__ __forceinline__ void part_ld8(const Partials& P, int64_t m, int64_t n, float (&r)[8]) {
  const float* q = P.p + m * P.ld + n;
  auto ld8 = [&](int z, float (&v)[8]) {
    const float4 a = *(const float4*)(q + (int64_t)z * P.stride), b = *(const float4*)(q + (int64_t)z * P.stride + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  };
  if (P.splits == 1) {
    ld8(0, r);
    return;
  }
  float s[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) s[u][i] = 0.f;
  int z = 0;
  for (; z + 4 <= P.splits; z += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) ld8(z + u, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) s[u][i] += v[u][i];
  }
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    if (z + u < P.splits) {
      float v[8];
      ld8(z + u, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[u][i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (s[0][i] + s[1][i]) + (s[2][i] + s[3][i]);
}

__host__ __device__ __forceinline__ bool part_vec8_ok(const Partials& P) {
  return ((uintptr_t)P.p & 15) == 0 && P.ld % 4 == 0 && (P.splits == 1 || P.stride % 4 == 0);
}

// ---- rotary tables and the layer-input RMSNorm ---------------------------------------
// inv_freq [dr/2] fp64: theta^(-2i/dr), or its YaRN blend when factor > 1.
hipError_t rope_inv_freq(int dr, double theta, double factor, int original_max_position, double beta_fast,
                         double beta_slow, double* inv_freq, hipStream_t s);
// cos/sin [n, dr/2] fp32 of (positions[t] (t if null) + pos_offset) * inv_freq[i]
// (theta = 10000 frequencies if inv_freq is null).
hipError_t rope_tables(int n, int dr, const int32_t* positions, int pos_offset, const double* inv_freq, float* cosT,
                       float* sinT, hipStream_t s);
// y [n, D] act = x * rsqrt(mean(x^2) + eps) * gamma per row.
hipError_t input_norm(const Dims& d, const void* x, int n, const float* gamma, void* y, hipStream_t s);

// ---- MX fp8 activation quantisation -------------------------------------------------
// Rows of x (bf16 [M, K], row stride ldx) per 128-column group: exponent e (E8M0 byte e+127)
// and E4M3FN codes of x * 2^-e.  With deq null: codes [M, K] and exps, either [ceil(K/128)][M]
// or, with exp_order, in the fp8 GEMM's f8_exp_order (rows padded to f8_rows_pad(M)).  With deq: only
// the dequantised bf16 values [M, K] (row stride K).
hipError_t quant_mx(const bf16_t* x, int64_t ldx, int M, int K, uint8_t* codes, uint8_t* exps, bool exp_order,
                    bf16_t* deq, hipStream_t s);

// ---- general (any shape) kernels: SIMT fp32 arithmetic ------------------------------
// C[M, N] fp32 (row stride ldc) = A[M, K] (act, row stride lda) @ W[K, N]
hipError_t gemm_simt(const Dims& d, const void* A, int64_t lda, const WeightView& W, float* C,
                     int64_t ldc, int M, int N, int K, hipStream_t s);

// Row builder.  Yq [T, *] holds cq (Lq columns, absent when Lq == 0), Ykv [T, *] holds
// [c_kv (Lkv) | k_pe (dr)].  Writes cqn = RMSNorm(cq)*gq (act [T, Lq], if non-null),
// cn = RMSNorm(c_kv)*gkv (act [T, Lkv], if non-null), the cache row [cn | RoPE(k_pe)] at
// slot_mapping[t] (if cache and slot_mapping are non-null), and K[t, h, dn:] = RoPE(k_pe)
// for every head (if kbuf is non-null).
hipError_t row_builder(const Dims& d, const Partials& Yq, const Partials& Ykv, int T, const float* gq,
                       const float* gkv, const float* cosT, const float* sinT, void* cqn, void* cn,
                       void* cache, int64_t n_slots, const int32_t* slot_mapping, void* kbuf,
                       hipStream_t s);

// q[t, h, :] (act) = [Y[t, h*dqk : h*dqk+dn] | RoPE(Y[t, h*dqk+dn : (h+1)*dqk])]
hipError_t q_epilogue(const Dims& d, const Partials& Y, int T, const float* cosT, const float* sinT, void* q,
                      hipStream_t s);

// KV[t, h*(dn+dv) + j] -> K[t, h, j] (j < dn) and V[t, h, j - dn] (act)
hipError_t kv_split(const Dims& d, const Partials& KV, int T, void* k, void* v, hipStream_t s);

// y (act, [M, N]) = Y
hipError_t cast_rows(const Dims& d, const Partials& Y, int M, int N, void* y, hipStream_t s);

// Absorbed decode, general version.  Qabs fp32 [B, H, R] = [q_nope @ W_UK | q_pe].
hipError_t fold_simt(const Dims& d, const void* q, int B, const WeightView& wkv_b, float* Qabs,
                     hipStream_t s);
// Split-context attention over the paged cache: partial (o_lat[Lkv], m, l) per
// (b, h, split) with split s covering tokens [s*chunk, (s+1)*chunk).  Query b reads
// its block ids from block_table + b * bt_stride (bt_stride 0: one table for all).
hipError_t decode_attn_simt(const Dims& d, const float* Qabs, int B, const void* cache,
                            int64_t n_blocks, const int32_t* block_table, int max_blocks,
                            int64_t bt_stride, const int32_t* ctx, int nsplit, int chunk, float* part_o,
                            float* part_ml, hipStream_t s);
// ctx[t] = prefix + t + 1 for t < T (the rows query t of a prefill chunk sees).
hipError_t chunk_ctx(int T, int prefix, int32_t* ctx, hipStream_t s);
// rows 0 .. N-1 of the sequence the block-table row `table` maps: latent parts into c [N, Lkv],
// rope parts broadcast into k [N, H, dqk] columns dn .. dqk (bf16, dims multiples of 8)
hipError_t chunk_gather(const Dims& d, const void* cache, int64_t n_blocks, const int32_t* table, int N, void* c,
                        void* k, hipStream_t s);
// Log-sum-exp merge of the splits, then o[b, h] = o_lat @ W_UV[h] (act).
hipError_t combine_simt(const Dims& d, int B, int nsplit, const float* part_o, const float* part_ml,
                        const WeightView& wkv_b, void* o, hipStream_t s);

// Causal flash attention, general version: q, k [T, H, dqk], v [T, H, dv] -> o [T, H, dv].
hipError_t prefill_attn_simt(const Dims& d, const void* q, const void* k, const void* v, int T,
                             void* o, hipStream_t s);

}  // namespace mla
