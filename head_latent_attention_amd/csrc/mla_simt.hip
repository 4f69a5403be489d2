// General-shape MLA kernels for gfx950 (SIMT fp32 arithmetic).
//
// These cover every shape the ABI accepts (including the fp32 activation path)
// and serve as the fallback where the MFMA kernels' shape constraints do not
// hold.  Each kernel is written for clarity first: fp32 accumulation, LDS tiling
// where it is cheap, no atomics, fixed reduction order (bitwise reproducible).
#include "mla_kernels.h"

namespace mla {

// ===================================================================================
// GEMM: C[M,N] = A[M,K] @ W[K,N], 64x64 tile, BK = 16, 256 threads, 4x4 per thread.
// ===================================================================================
template <typename TA, int WK>
__global__ __launch_bounds__(256) void gemm_simt_kernel(const TA* __restrict__ A, int64_t lda,
                                                        WeightView W, float* __restrict__ C,
                                                        int64_t ldc, int M, int N, int K) {
  __shared__ float As[16][65];
  __shared__ float Ws[16][64];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid + 256 * i;
      int r = e >> 4, kk = e & 15;
      int m = m0 + r, k = k0 + kk;
      As[kk][r] = (m < M && k < K) ? Act<TA>::ld(A, (size_t)m * lda + k) : 0.f;
      int kw = e >> 6, nn = e & 63;
      int n = n0 + nn, k2 = k0 + kw;
      Ws[kw][nn] = (n < N && k2 < K) ? load_w<WK>(W, k2, n) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Ws[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + ty + 16 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int n = n0 + tx + 16 * j;
      if (n < N) C[(size_t)m * ldc + n] = acc[i][j];
    }
  }
}

template <typename TA>
static hipError_t gemm_simt_t(const Dims& d, const void* A, int64_t lda, const WeightView& W,
                              float* C, int64_t ldc, int M, int N, int K, hipStream_t s) {
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  switch (d.wk) {
    case W_F32: gemm_simt_kernel<TA, W_F32><<<grid, 256, 0, s>>>((const TA*)A, lda, W, C, ldc, M, N, K); break;
    case W_BF16: gemm_simt_kernel<TA, W_BF16><<<grid, 256, 0, s>>>((const TA*)A, lda, W, C, ldc, M, N, K); break;
    default: gemm_simt_kernel<TA, W_FP8><<<grid, 256, 0, s>>>((const TA*)A, lda, W, C, ldc, M, N, K); break;
  }
  return hipGetLastError();
}

hipError_t gemm_simt(const Dims& d, const void* A, int64_t lda, const WeightView& W, float* C,
                     int64_t ldc, int M, int N, int K, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  return d.act == 0 ? gemm_simt_t<float>(d, A, lda, W, C, ldc, M, N, K, s)
                    : gemm_simt_t<bf16_t>(d, A, lda, W, C, ldc, M, N, K, s);
}

// ===================================================================================
// Row builder: RMSNorm of both latents, RoPE of k_pe, cache-row scatter, k_pe broadcast.
// Grid (tokens, 2): y = 0 normalises the query latent, y = 1 builds the kv row.
// ===================================================================================
// Each thread keeps up to kRowCache of its values in registers between the two passes of
// the RMSNorm (longer rows are read again).
constexpr int kRowCache = 4;

template <typename T>
__global__ __launch_bounds__(512) void row_builder_kernel(
    Partials Yq, Partials Ykv, int Lq, int Lkv, int dr, const float* __restrict__ gq, const float* __restrict__ gkv, float eps,
    const float* __restrict__ cosT, const float* __restrict__ sinT, T* __restrict__ cqn, T* __restrict__ cn,
    T* __restrict__ cache, int64_t n_slots, const int32_t* __restrict__ slot_mapping, T* __restrict__ kbuf, int H,
    int dn) {
  __shared__ float red[16];
  __shared__ __attribute__((aligned(16))) float kpe_row[256];  // dr <= 256 elements (fp32 or bf16)
  const int t = blockIdx.x;
  const int R = Lkv + dr, dqk = dn + dr;
  const int nt = blockDim.x;
  float v[kRowCache];
  if (blockIdx.y == 0) {
    // query latent: RMSNorm(cq) * gq
    if (Lq == 0 || cqn == nullptr) return;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < kRowCache; ++c) {
      const int i = threadIdx.x + c * nt;
      v[c] = i < Lq ? part_ld(Yq, t, i) : 0.f;
      ss += v[c] * v[c];
    }
    for (int i = threadIdx.x + kRowCache * nt; i < Lq; i += nt) {
      const float x = part_ld(Yq, t, i);
      ss += x * x;
    }
    const float r = rsqrtf(block_sum(ss, red) / (float)Lq + eps);
#pragma unroll
    for (int c = 0; c < kRowCache; ++c) {
      const int i = threadIdx.x + c * nt;
      if (i < Lq) Act<T>::st(cqn, (size_t)t * Lq + i, v[c] * r * gq[i]);
    }
    for (int i = threadIdx.x + kRowCache * nt; i < Lq; i += nt)
      Act<T>::st(cqn, (size_t)t * Lq + i, part_ld(Yq, t, i) * r * gq[i]);
    return;
  }
  // kv latent: RMSNorm(c_kv) * gkv, RoPE(k_pe), cache row, k_pe broadcast
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kRowCache; ++c) {
    const int i = threadIdx.x + c * nt;
    v[c] = i < Lkv ? part_ld(Ykv, t, i) : 0.f;
    ss += v[c] * v[c];
  }
  for (int i = threadIdx.x + kRowCache * nt; i < Lkv; i += nt) {
    const float x = part_ld(Ykv, t, i);
    ss += x * x;
  }
  const float r = rsqrtf(block_sum(ss, red) / (float)Lkv + eps);
  int64_t slot = -1;
  if (cache != nullptr && slot_mapping != nullptr) {
    slot = slot_mapping[t];
    if (slot >= n_slots) slot = -1;
  }
  auto put = [&](int i, float x) {
    const float y = Act<T>::round(x * r * gkv[i]);
    if (cn) Act<T>::st(cn, (size_t)t * Lkv + i, y);
    if (slot >= 0) Act<T>::st(cache, (size_t)slot * R + i, y);
  };
#pragma unroll
  for (int c = 0; c < kRowCache; ++c) {
    const int i = threadIdx.x + c * nt;
    if (i < Lkv) put(i, v[c]);
  }
  for (int i = threadIdx.x + kRowCache * nt; i < Lkv; i += nt) put(i, part_ld(Ykv, t, i));
  const int half = dr >> 1;
  T* kpe = (T*)kpe_row;  // the roped k_pe of this token, for the broadcast below
  for (int i = threadIdx.x; i < half; i += nt) {
    const float c = cosT[(size_t)t * half + i], sn = sinT[(size_t)t * half + i];
    const float x0 = part_ld(Ykv, t, Lkv + 2 * i), x1 = part_ld(Ykv, t, Lkv + 2 * i + 1);
    const float y0 = Act<T>::round(x0 * c - x1 * sn), y1 = Act<T>::round(x0 * sn + x1 * c);
    if (slot >= 0) {
      Act<T>::st(cache, (size_t)slot * R + Lkv + 2 * i, y0);
      Act<T>::st(cache, (size_t)slot * R + Lkv + 2 * i + 1, y1);
    }
    if (kbuf) {
      Act<T>::st(kpe, 2 * i, y0);
      Act<T>::st(kpe, 2 * i + 1, y1);
    }
  }
  if (!kbuf) return;
  // k_pe broadcast into every head's key: k[t, h, dn : dn + dr] = k_pe.  With 16-byte aligned
  // head slices every thread writes whole 16-byte chunks (H * dr / chunk stores per token);
  // otherwise one element per thread and step.
  __syncthreads();
  constexpr int kPer = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  T* krow = kbuf + (size_t)t * H * dqk + dn;
  if (dr % kPer == 0 && dqk % kPer == 0 && dn % kPer == 0 && ((uintptr_t)kbuf & 15) == 0) {
    const int cpr = dr / kPer;  // chunks per head
    for (int e = threadIdx.x; e < H * cpr; e += nt) {
      const int h = e / cpr, c = e - h * cpr;
      *(uint4*)(krow + (size_t)h * dqk + c * kPer) = *(const uint4*)(kpe + c * kPer);
    }
  } else {
    for (int e = threadIdx.x; e < H * dr; e += nt) {
      const int h = e / dr, i = e - h * dr;
      krow[(size_t)h * dqk + i] = kpe[i];
    }
  }
}

// bf16 rows with every width a multiple of 8: one 256-thread workgroup per token, each thread
// handling up to MAXC 8-column chunks of [q latent | kv latent | k_pe] (16-byte partial loads in
// part_ld's order, both sums of squares in one block reduction, 16-byte stores), the roped k_pe
// staged in LDS for the per-head broadcast.
template <int MAXC>
__global__ __launch_bounds__(256) void row_builder_bf16x8_kernel(
    Partials Yq, Partials Ykv, int Lq, int Lkv, int dr, const float* __restrict__ gq, const float* __restrict__ gkv,
    float eps, const float* __restrict__ cosT, const float* __restrict__ sinT, bf16_t* __restrict__ cqn,
    bf16_t* __restrict__ cn, bf16_t* __restrict__ cache, int64_t n_slots, const int32_t* __restrict__ slot_mapping,
    bf16_t* __restrict__ kbuf, int H, int dn) {
  __shared__ float red[2][4];
  __shared__ __attribute__((aligned(16))) uint4 kpe_s[32];  // dr <= 256
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nq = Lq / 8, nk = Lkv / 8, nr = dr / 8, total = nq + nk + nr;
  const int R = Lkv + dr, dqk = dn + dr, half = dr >> 1;
  // grid y = 2: workgroup y takes the query latent (y = 0) or the kv latent and rope key (y = 1)
  // of its row, so that two workgroups share the row's partial sums; y = 1: all of them
  const int e_lo = gridDim.y == 2 && blockIdx.y == 1 ? nq : 0;
  const int e_hi = gridDim.y == 2 && blockIdx.y == 0 ? nq : total;
  float v[MAXC][8];
  float ssq = 0.f, ssk = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = e_lo + tid + 256 * c;
    if (e >= e_hi) {
    } else if (e < nq) {
      part_ld8(Yq, t, 8 * e, v[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ssq += v[c][i] * v[c][i];
    } else if (e < nq + nk) {
      part_ld8(Ykv, t, 8 * (e - nq), v[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ssk += v[c][i] * v[c][i];
    } else if (e < total) {
      part_ld8(Ykv, t, Lkv + 8 * (e - nq - nk), v[c]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ssq += __shfl_xor(ssq, off);
    ssk += __shfl_xor(ssk, off);
  }
  if (lane == 0) {
    red[0][w] = ssq;
    red[1][w] = ssk;
  }
  __syncthreads();
  const float rq = nq > 0 ? rsqrtf(((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) / (float)Lq + eps) : 0.f;
  const float rk = rsqrtf(((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) / (float)Lkv + eps);
  int64_t slot = -1;
  if (cache != nullptr && slot_mapping != nullptr) {
    slot = slot_mapping[t];
    if (slot >= n_slots) slot = -1;
  }
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = e_lo + tid + 256 * c;
    float y[8];
    if (e >= e_hi) {
    } else if (e < nq) {
      if (!cqn) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = v[c][i] * rq * gq[8 * e + i];
      *(uint4*)(cqn + t * Lq + 8 * e) =
          make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
    } else if (e < nq + nk) {
      const int i0 = 8 * (e - nq);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = v[c][i] * rk * gkv[i0 + i];
      const uint4 pk =
          make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
      if (cn) *(uint4*)(cn + t * Lkv + i0) = pk;
      if (slot >= 0) *(uint4*)(cache + slot * R + i0) = pk;
    } else if (e < total) {
      const int ch = e - nq - nk, p0 = 4 * ch;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float cs = cosT[t * half + p0 + i], sn = sinT[t * half + p0 + i];
        const float x0 = v[c][2 * i], x1 = v[c][2 * i + 1];
        y[2 * i] = x0 * cs - x1 * sn;
        y[2 * i + 1] = x0 * sn + x1 * cs;
      }
      const uint4 pk =
          make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
      if (slot >= 0) *(uint4*)(cache + slot * R + Lkv + 8 * ch) = pk;
      kpe_s[ch] = pk;
    }
  }
  if (!kbuf || e_hi < total) return;
  __syncthreads();
  bf16_t* krow = kbuf + t * H * dqk + dn;
  for (int e = tid; e < H * nr; e += 256) {
    const int h = e / nr, c = e - h * nr;
    *(uint4*)(krow + (int64_t)h * dqk + 8 * c) = kpe_s[c];
  }
}

hipError_t row_builder(const Dims& d, const Partials& Yq, const Partials& Ykv, int T, const float* gq, const float* gkv, const float* cosT,
                       const float* sinT, void* cqn, void* cn, void* cache, int64_t n_slots,
                       const int32_t* slot_mapping, void* kbuf, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int total8 = (d.Lq + d.Lkv + d.dr) / 8;
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (d.act == 1 && d.Lq % 8 == 0 && d.Lkv % 8 == 0 && d.dr % 8 == 0 && d.dn % 8 == 0 && d.dr <= 256 &&
      total8 <= 512 && (d.Lq == 0 || part_vec8_ok(Yq)) && part_vec8_ok(Ykv) && al16(cqn) && al16(cn) && al16(cache) &&
      al16(kbuf)) {
    // two workgroups per row (query latent; kv latent and rope key) when each part fits one pass
    const bool split = d.Lq > 0 && d.Lq / 8 <= 256 && (d.Lkv + d.dr) / 8 <= 256;
    if (split)
      row_builder_bf16x8_kernel<1><<<dim3(T, 2), 256, 0, s>>>(Yq, Ykv, d.Lq, d.Lkv, d.dr, gq, gkv, d.eps, cosT, sinT,
                                                              (bf16_t*)cqn, (bf16_t*)cn, (bf16_t*)cache, n_slots,
                                                              slot_mapping, (bf16_t*)kbuf, d.H, d.dn);
    else if (total8 <= 256)
      row_builder_bf16x8_kernel<1><<<T, 256, 0, s>>>(Yq, Ykv, d.Lq, d.Lkv, d.dr, gq, gkv, d.eps, cosT, sinT,
                                                     (bf16_t*)cqn, (bf16_t*)cn, (bf16_t*)cache, n_slots, slot_mapping,
                                                     (bf16_t*)kbuf, d.H, d.dn);
    else
      row_builder_bf16x8_kernel<2><<<T, 256, 0, s>>>(Yq, Ykv, d.Lq, d.Lkv, d.dr, gq, gkv, d.eps, cosT, sinT,
                                                     (bf16_t*)cqn, (bf16_t*)cn, (bf16_t*)cache, n_slots, slot_mapping,
                                                     (bf16_t*)kbuf, d.H, d.dn);
    return hipGetLastError();
  }
  dim3 grid(T, 2);
  if (d.act == 0)
    row_builder_kernel<float><<<grid, 512, 0, s>>>(Yq, Ykv, d.Lq, d.Lkv, d.dr, gq, gkv, d.eps, cosT, sinT, (float*)cqn,
                                                    (float*)cn, (float*)cache, n_slots, slot_mapping, (float*)kbuf,
                                                    d.H, d.dn);
  else
    row_builder_kernel<bf16_t><<<grid, 512, 0, s>>>(Yq, Ykv, d.Lq, d.Lkv, d.dr, gq, gkv, d.eps, cosT, sinT, (bf16_t*)cqn,
                                                     (bf16_t*)cn, (bf16_t*)cache, n_slots, slot_mapping,
                                                     (bf16_t*)kbuf, d.H, d.dn);
  return hipGetLastError();
}

// ===================================================================================
// Query epilogue: per-head RoPE on the trailing dr dims and the cast to act.
// ===================================================================================
template <typename T>
__global__ __launch_bounds__(256) void q_epilogue_kernel(Partials Y, int H, int dn, int dr,
                                                         const float* __restrict__ cosT,
                                                         const float* __restrict__ sinT, T* __restrict__ q) {
  // one thread per (token, head, rope pair or nope element); grid (T, ceil(H * (dn + dr/2) / 256))
  const int t = blockIdx.x, dqk = dn + dr, half = dr >> 1, per_head = dn + half;
  const int e = blockIdx.y * blockDim.x + threadIdx.x;
  if (e >= H * per_head) return;
  const int h = e / per_head, u = e - h * per_head;
  const size_t o = (size_t)t * H * dqk + (size_t)h * dqk;
  if (u < dn) {
    Act<T>::st(q, o + u, part_ld(Y, t, (int64_t)h * dqk + u));
  } else {
    const int i = u - dn;
    const float c = cosT[(size_t)t * half + i], sn = sinT[(size_t)t * half + i];
    const float x0 = part_ld(Y, t, (int64_t)h * dqk + dn + 2 * i), x1 = part_ld(Y, t, (int64_t)h * dqk + dn + 2 * i + 1);
    Act<T>::st(q, o + dn + 2 * i, x0 * c - x1 * sn);
    Act<T>::st(q, o + dn + 2 * i + 1, x0 * sn + x1 * c);
  }
}

// bf16 queries with dn and dr multiples of 8: one thread per 8 consecutive columns (16-byte
// partial loads, one 16-byte store); a chunk in the rope part holds four whole pairs.
__global__ __launch_bounds__(256) void q_epilogue_bf16x8_kernel(Partials Y, int64_t chunks, int H, int dn, int dr,
                                                                const float* __restrict__ cosT,
                                                                const float* __restrict__ sinT, bf16_t* __restrict__ q) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= chunks) return;
  const int dqk = dn + dr, half = dr >> 1, per_row = H * dqk / 8;
  const int64_t t = e / per_row;
  const int n = 8 * (int)(e - t * per_row), h = n / dqk, u = n - h * dqk;
  float v[8];
  part_ld8(Y, t, n, v);
  if (u >= dn) {
    const int p0 = (u - dn) >> 1;
    const float4 c4 = *(const float4*)(cosT + t * half + p0), s4 = *(const float4*)(sinT + t * half + p0);
    const float c[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = v[2 * i], x1 = v[2 * i + 1];
      v[2 * i] = x0 * c[i] - x1 * sn[i];
      v[2 * i + 1] = x0 * sn[i] + x1 * c[i];
    }
  }
  *(uint4*)(q + t * H * dqk + n) =
      make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

hipError_t q_epilogue(const Dims& d, const Partials& Y, int T, const float* cosT, const float* sinT, void* q,
                      hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d.act == 1 && d.dn % 8 == 0 && d.dr % 8 == 0 && part_vec8_ok(Y) && ((uintptr_t)cosT & 15) == 0 &&
      ((uintptr_t)sinT & 15) == 0 && ((uintptr_t)q & 15) == 0) {
    const int64_t chunks = (int64_t)T * d.H * (d.dn + d.dr) / 8;
    q_epilogue_bf16x8_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, s>>>(Y, chunks, d.H, d.dn, d.dr, cosT, sinT,
                                                                               (bf16_t*)q);
    return hipGetLastError();
  }
  dim3 grid(T, (d.H * (d.dn + d.dr / 2) + 255) / 256);
  if (d.act == 0) q_epilogue_kernel<float><<<grid, 256, 0, s>>>(Y, d.H, d.dn, d.dr, cosT, sinT, (float*)q);
  else q_epilogue_kernel<bf16_t><<<grid, 256, 0, s>>>(Y, d.H, d.dn, d.dr, cosT, sinT, (bf16_t*)q);
  return hipGetLastError();
}

// ===================================================================================
// KV split: [k_nope | v] per head -> K[..., :dn], V.
// ===================================================================================
template <typename T>
__global__ __launch_bounds__(256) void kv_split_kernel(Partials KV, int H, int dn, int dr, int dv, T* __restrict__ k,
                                                       T* __restrict__ v) {
  const int t = blockIdx.x, w = dn + dv, dqk = dn + dr;
  const int e = blockIdx.y * blockDim.x + threadIdx.x;
  if (e >= H * w) return;
  const int h = e / w, j = e - h * w;
  const float x = part_ld(KV, t, e);
  if (j < dn) Act<T>::st(k, ((size_t)t * H + h) * dqk + j, x);
  else Act<T>::st(v, ((size_t)t * H + h) * dv + (j - dn), x);
}

hipError_t kv_split(const Dims& d, const Partials& KV, int T, void* k, void* v, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dim3 grid(T, (d.H * (d.dn + d.dv) + 255) / 256);
  if (d.act == 0) kv_split_kernel<float><<<grid, 256, 0, s>>>(KV, d.H, d.dn, d.dr, d.dv, (float*)k, (float*)v);
  else kv_split_kernel<bf16_t><<<grid, 256, 0, s>>>(KV, d.H, d.dn, d.dr, d.dv, (bf16_t*)k, (bf16_t*)v);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(Partials Y, int M, int N, T* __restrict__ y) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / N, n = i - m * N;
    Act<T>::st(y, i, part_ld(Y, m, n));
  }
}

// bf16 rows with N a multiple of 8: one thread per 8 consecutive columns.
__global__ __launch_bounds__(256) void cast_bf16x8_kernel(Partials Y, int64_t chunks, int N, bf16_t* __restrict__ y) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= chunks) return;
  const int64_t m = (8 * e) / N, n = 8 * e - m * N;
  float v[8];
  part_ld8(Y, m, n, v);
  *(uint4*)(y + 8 * e) =
      make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

hipError_t cast_rows(const Dims& d, const Partials& Y, int M, int N, void* y, hipStream_t s) {
  const int64_t n = (int64_t)M * N;
  if (n <= 0) return hipSuccess;
  if (d.act == 1 && N % 8 == 0 && part_vec8_ok(Y) && ((uintptr_t)y & 15) == 0) {
    const int64_t chunks = n / 8;
    cast_bf16x8_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, s>>>(Y, chunks, N, (bf16_t*)y);
    return hipGetLastError();
  }
  const int grid = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  if (d.act == 0) cast_kernel<float><<<grid, 256, 0, s>>>(Y, M, N, (float*)y);
  else cast_kernel<bf16_t><<<grid, 256, 0, s>>>(Y, M, N, (bf16_t*)y);
  return hipGetLastError();
}

// ===================================================================================
// Absorbed decode, general kernels.
// ===================================================================================
template <typename T, int WK>
__global__ __launch_bounds__(256) void fold_simt_kernel(const T* __restrict__ q, int H, int dn, int dr,
                                                        int dv, int Lkv, WeightView W,
                                                        float* __restrict__ Qabs) {
  extern __shared__ float qn[];
  const int bh = blockIdx.x, h = bh % H;
  const int dqk = dn + dr, R = Lkv + dr;
  const T* qrow = q + (size_t)bh * dqk;
  for (int p = threadIdx.x; p < dn; p += blockDim.x) qn[p] = Act<T>::ld(qrow, p);
  __syncthreads();
  const int64_t col0 = (int64_t)h * (dn + dv);
  for (int c = threadIdx.x; c < Lkv; c += blockDim.x) {
    float acc = 0.f;
    for (int p = 0; p < dn; ++p) acc = fmaf(qn[p], load_w<WK>(W, c, col0 + p), acc);
    Qabs[(size_t)bh * R + c] = acc;
  }
  for (int i = threadIdx.x; i < dr; i += blockDim.x) Qabs[(size_t)bh * R + Lkv + i] = Act<T>::ld(qrow, dn + i);
}

hipError_t fold_simt(const Dims& d, const void* q, int B, const WeightView& W, float* Qabs, hipStream_t s) {
  const int grid = B * d.H;
  const size_t sh = sizeof(float) * d.dn;
#define FOLD_LAUNCH(T, WK) fold_simt_kernel<T, WK><<<grid, 256, sh, s>>>((const T*)q, d.H, d.dn, d.dr, d.dv, d.Lkv, W, Qabs)
  if (d.act == 0) FOLD_LAUNCH(float, W_F32);
  else if (d.wk == W_BF16) FOLD_LAUNCH(bf16_t, W_BF16);
  else FOLD_LAUNCH(bf16_t, W_FP8);
#undef FOLD_LAUNCH
  return hipGetLastError();
}

// One block per (b, h, split); 256 threads; tokens processed in tiles of 256.
template <typename T>
__global__ __launch_bounds__(256) void decode_attn_simt_kernel(
    const float* __restrict__ Qabs, int H, int Lkv, int dr, float scale, const T* __restrict__ cache,
    int64_t n_blocks, int bs, const int32_t* __restrict__ block_table, int max_blocks, int64_t bt_stride,
    const int32_t* __restrict__ ctx_lens, int nsplit, int chunk, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  extern __shared__ float sh[];
  const int R = Lkv + dr;
  float* Q = sh;             // [R]
  float* P = sh + R;         // [256]
  __shared__ float red[16];
  __shared__ int64_t rowoff[256];
  const int bh = blockIdx.x, sidx = blockIdx.y, b = bh / H;
  for (int i = threadIdx.x; i < R; i += blockDim.x) Q[i] = Qabs[(size_t)bh * R + i];
  const int ctx = ctx_lens[b];
  const int t0 = sidx * chunk, t1 = min(ctx, t0 + chunk);
  float m = -INFINITY, l = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};  // c = threadIdx.x + 256*j, Lkv <= 1024
  __syncthreads();
  for (int tb = t0; tb < t1; tb += 256) {
    const int t = tb + threadIdx.x;
    float sc = -INFINITY;
    int64_t off = -1;
    if (t < t1 && t / bs < max_blocks) {
      const int blk = block_table[(size_t)b * bt_stride + t / bs];
      if (blk >= 0 && blk < n_blocks) {
        off = ((int64_t)blk * bs + (t % bs)) * R;
        float acc = 0.f;
        for (int dd = 0; dd < R; ++dd) acc = fmaf(Q[dd], Act<T>::ld(cache, off + dd), acc);
        sc = acc * scale;
      }
    }
    rowoff[threadIdx.x] = off;
    const float tmax = block_max(sc, red);
    const float mnew = fmaxf(m, tmax);
    const float p = (sc == -INFINITY) ? 0.f : __expf(sc - mnew);
    P[threadIdx.x] = p;
    const float psum = block_sum(p, red);  // contains __syncthreads before reads of P / rowoff
    const float corr = (m == -INFINITY) ? 0.f : __expf(m - mnew);
    l = l * corr + psum;
    m = mnew;
    const int nt = min(256, t1 - tb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + 256 * j;
      if (c >= Lkv) break;
      float acc = o[j] * corr;
      for (int u = 0; u < nt; ++u) {
        const int64_t ro = rowoff[u];
        if (ro >= 0) acc = fmaf(P[u], Act<T>::ld(cache, ro + c), acc);
      }
      o[j] = acc;
    }
    __syncthreads();
  }
  const size_t pidx = (size_t)bh * nsplit + sidx;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < Lkv) part_o[pidx * Lkv + c] = o[j];
  }
  if (threadIdx.x == 0) {
    part_ml[pidx * 2] = m;
    part_ml[pidx * 2 + 1] = l;
  }
}

hipError_t decode_attn_simt(const Dims& d, const float* Qabs, int B, const void* cache, int64_t n_blocks,
                            const int32_t* block_table, int max_blocks, int64_t bt_stride, const int32_t* ctx,
                            int nsplit, int chunk, float* part_o, float* part_ml, hipStream_t s) {
  dim3 grid(B * d.H, nsplit);
  const size_t sh = sizeof(float) * (d.R() + 256);
  if (d.act == 0)
    decode_attn_simt_kernel<float><<<grid, 256, sh, s>>>(Qabs, d.H, d.Lkv, d.dr, d.scale, (const float*)cache,
                                                          n_blocks, d.bs, block_table, max_blocks, bt_stride, ctx,
                                                          nsplit, chunk, part_o, part_ml);
  else
    decode_attn_simt_kernel<bf16_t><<<grid, 256, sh, s>>>(Qabs, d.H, d.Lkv, d.dr, d.scale, (const bf16_t*)cache,
                                                           n_blocks, d.bs, block_table, max_blocks, bt_stride, ctx,
                                                           nsplit, chunk, part_o, part_ml);
  return hipGetLastError();
}

template <typename T, int WK>
__global__ __launch_bounds__(256) void combine_simt_kernel(int H, int Lkv, int dn, int dv, int nsplit,
                                                           const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           WeightView W, T* __restrict__ o) {
  extern __shared__ float ol[];  // [Lkv]
  const int bh = blockIdx.x, h = bh % H;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = part_ml[((size_t)bh * nsplit + s) * 2];
    M = fmaxf(M, ms);
  }
  float L = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = part_ml[((size_t)bh * nsplit + s) * 2], ls = part_ml[((size_t)bh * nsplit + s) * 2 + 1];
    if (ms != -INFINITY) L += ls * __expf(ms - M);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int c = threadIdx.x; c < Lkv; c += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float ms = part_ml[((size_t)bh * nsplit + s) * 2];
      if (ms != -INFINITY) acc += part_o[((size_t)bh * nsplit + s) * Lkv + c] * __expf(ms - M);
    }
    ol[c] = acc * inv;
  }
  __syncthreads();
  const int64_t col0 = (int64_t)h * (dn + dv) + dn;
  for (int j = threadIdx.x; j < dv; j += blockDim.x) {
    float acc = 0.f;
    for (int c = 0; c < Lkv; ++c) acc = fmaf(ol[c], load_w<WK>(W, c, col0 + j), acc);
    Act<T>::st(o, (size_t)bh * dv + j, acc);
  }
}

hipError_t combine_simt(const Dims& d, int B, int nsplit, const float* part_o, const float* part_ml,
                        const WeightView& W, void* o, hipStream_t s) {
  const int grid = B * d.H;
  const size_t sh = sizeof(float) * d.Lkv;
#define COMB_LAUNCH(T, WK) combine_simt_kernel<T, WK><<<grid, 256, sh, s>>>(d.H, d.Lkv, d.dn, d.dv, nsplit, part_o, part_ml, W, (T*)o)
  if (d.act == 0) COMB_LAUNCH(float, W_F32);
  else if (d.wk == W_BF16) COMB_LAUNCH(bf16_t, W_BF16);
  else COMB_LAUNCH(bf16_t, W_FP8);
#undef COMB_LAUNCH
  return hipGetLastError();
}

// ===================================================================================
// Causal prefill attention, general version.  Block = 16 queries x 16 lanes of one
// head; key tiles of 32 staged in LDS as fp32; online softmax.
// ===================================================================================
template <typename T>
__global__ __launch_bounds__(256) void prefill_attn_simt_kernel(const T* __restrict__ q,
                                                                const T* __restrict__ k,
                                                                const T* __restrict__ v, int T_, int H,
                                                                int dqk, int dv, float scale,
                                                                T* __restrict__ o) {
  extern __shared__ float sh[];
  float* Qs = sh;                    // [16][dqk]
  float* Ks = Qs + 16 * dqk;         // [32][dqk + 1]
  float* Vs = Ks + 32 * (dqk + 1);   // [32][dv]
  float* Ps = Vs + 32 * dv;          // [16][32]
  const int h = blockIdx.y, q0 = blockIdx.x * 16;
  const int tid = threadIdx.x, qi = tid >> 4, lane = tid & 15;
  const int tq = q0 + qi;
  for (int e = tid; e < 16 * dqk; e += 256) {
    const int r = e / dqk, c = e - r * dqk;
    Qs[e] = (q0 + r < T_) ? Act<T>::ld(q, ((size_t)(q0 + r) * H + h) * dqk + c) : 0.f;
  }
  float m = -INFINITY, l = 0.f;
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
  const int kend = min(T_, q0 + 16);  // causal: keys < kend
  for (int k0 = 0; k0 < kend; k0 += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * dqk; e += 256) {
      const int r = e / dqk, c = e - r * dqk;
      Ks[r * (dqk + 1) + c] = (k0 + r < T_) ? Act<T>::ld(k, ((size_t)(k0 + r) * H + h) * dqk + c) : 0.f;
    }
    for (int e = tid; e < 32 * dv; e += 256) {
      const int r = e / dv, c = e - r * dv;
      Vs[e] = (k0 + r < T_) ? Act<T>::ld(v, ((size_t)(k0 + r) * H + h) * dv + c) : 0.f;
    }
    __syncthreads();
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kj = lane + 16 * u, tk = k0 + kj;
      float a = 0.f;
      for (int c = 0; c < dqk; ++c) a = fmaf(Qs[qi * dqk + c], Ks[kj * (dqk + 1) + c], a);
      s[u] = (tk <= tq && tq < T_) ? a * scale : -INFINITY;
    }
    float tmax = fmaxf(s[0], s[1]);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, 16));
    const float mnew = fmaxf(m, tmax);
    float p0 = (s[0] == -INFINITY) ? 0.f : __expf(s[0] - mnew);
    float p1 = (s[1] == -INFINITY) ? 0.f : __expf(s[1] - mnew);
    Ps[qi * 32 + lane] = p0;
    Ps[qi * 32 + lane + 16] = p1;
    float ps = p0 + p1;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) ps += __shfl_xor(ps, off, 16);
    const float corr = (m == -INFINITY) ? 0.f : __expf(m - mnew);
    l = l * corr + ps;
    m = mnew;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = lane + 16 * j;
      if (c < dv) {
        float a = acc[j] * corr;
        for (int kj = 0; kj < 32; ++kj) a = fmaf(Ps[qi * 32 + kj], Vs[kj * dv + c], a);
        acc[j] = a;
      }
    }
  }
  if (tq < T_) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = lane + 16 * j;
      if (c < dv) Act<T>::st(o, ((size_t)tq * H + h) * dv + c, acc[j] * inv);
    }
  }
}

hipError_t prefill_attn_simt(const Dims& d, const void* q, const void* k, const void* v, int T, void* o,
                             hipStream_t s) {
  dim3 grid((T + 15) / 16, d.H);
  const int dqk = d.dqk();
  const size_t sh = sizeof(float) * (16 * dqk + 32 * (dqk + 1) + 32 * d.dv + 16 * 32);
  // set on every call: the attribute is per device and the call is host-side only
  const void* fn = d.act == 0 ? (const void*)prefill_attn_simt_kernel<float> : (const void*)prefill_attn_simt_kernel<bf16_t>;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
  if (e != hipSuccess) return e;
  if (d.act == 0)
    prefill_attn_simt_kernel<float><<<grid, 256, sh, s>>>((const float*)q, (const float*)k, (const float*)v, T,
                                                           d.H, dqk, d.dv, d.scale, (float*)o);
  else
    prefill_attn_simt_kernel<bf16_t><<<grid, 256, sh, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                                                            T, d.H, dqk, d.dv, d.scale, (bf16_t*)o);
  return hipGetLastError();
}

// Context length of each query of a prefill chunk: query t at position prefix + t sees
// prefix + t + 1 rows.
__global__ void chunk_ctx_kernel(int T, int prefix, int32_t* __restrict__ ctx) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) ctx[t] = prefix + t + 1;
}

hipError_t chunk_ctx(int T, int prefix, int32_t* ctx, hipStream_t s) {
  chunk_ctx_kernel<<<(T + 255) / 256, 256, 0, s>>>(T, prefix, ctx);
  return hipGetLastError();
}

// Rows 0 .. N-1 of one sequence's paged cache for the expanded chunk attention: the latent part
// of row r into c[r] (Lkv values), its rope part into k[r, h, dn:dqk] for every head (the rope
// key is shared by all heads).  One workgroup per row; rows whose block id is out of range are
// zero.  bf16 rows; Lkv, dr, dn multiples of 8.
__global__ __launch_bounds__(256) void chunk_gather_kernel(const bf16_t* __restrict__ cache, int64_t n_blocks, int bs,
                                                           const int32_t* __restrict__ table, int Lkv, int dr, int H,
                                                           int dn, bf16_t* __restrict__ c, bf16_t* __restrict__ k) {
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x;
  const int blk = table[r / bs];
  const bool ok = blk >= 0 && blk < n_blocks;
  const bf16_t* src = cache + ((int64_t)(ok ? blk : 0) * bs + r % bs) * (Lkv + dr);
  const int lc = Lkv / 8, pc = dr / 8, dqk = dn + dr;
  for (int i = t; i < lc; i += 256)
    *(uint4*)(c + r * Lkv + 8 * i) = ok ? *(const uint4*)(src + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
  // rope chunk t % pc of every head h = t / pc, t / pc + 256 / pc, ...
  const int ch = t % pc, hstep = 256 / pc;
  if (t >= hstep * pc) return;
  const uint4 v = ok ? *(const uint4*)(src + Lkv + 8 * ch) : make_uint4(0u, 0u, 0u, 0u);
  for (int h = t / pc; h < H; h += hstep) *(uint4*)(k + (r * H + h) * dqk + dn + 8 * ch) = v;
}

hipError_t chunk_gather(const Dims& d, const void* cache, int64_t n_blocks, const int32_t* table, int N, void* c,
                        void* k, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  chunk_gather_kernel<<<N, 256, 0, s>>>((const bf16_t*)cache, n_blocks, d.bs, table, d.Lkv, d.dr, d.H, d.dn,
                                        (bf16_t*)c, (bf16_t*)k);
  return hipGetLastError();
}

}  // namespace mla
