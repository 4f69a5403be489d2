// MFMA (CDNA4 matrix core) kernels for the shapes of the V2/V3 configurations.
// Each entry point reports whether it supports a shape; the general kernels in
// mla_simt.hip handle everything else.
#pragma once
#include "mla_kernels.h"

namespace mla {

struct FastDecodeWs {
  void* base = nullptr;
  size_t bytes = 0;
};

// Projection GEMM / GEMV: C[M, N] = A[M, K] (act) @ [W0 | W1], W0 giving output columns
// [0, n_split) and W1 columns [n_split, N) (n_split >= N: W0 only).  C is left in `out`
// (fast_gemm_out_bytes(M, N, K) bytes) as split-K partial sums, described by *res.
bool fast_proj_supported(const Dims& d);
size_t fast_gemm_out_bytes(int M, int N, int K);
hipError_t fast_gemm(const Dims& d, const void* A, int64_t lda, const WeightView& W0, int n_split,
                     const WeightView& W1, int M, int N, int K, float* out, Partials* res, hipStream_t s);

// Absorbed decode: fold, split-context attention over the paged cache, combine with W_UV.
bool fast_decode_supported(const Dims& d);
size_t fast_decode_ws_bytes(const Dims& d, int B, int max_context);
hipError_t fast_decode_attn(const Dims& d, const void* q, int B, const void* cache, int64_t n_blocks,
                            const int32_t* block_table, int max_blocks, const int32_t* ctx,
                            const WeightView& wkv_b, void* o, const FastDecodeWs& ws, hipStream_t s);

// Causal prefill flash attention.
bool fast_prefill_attn_supported(const Dims& d);
size_t fast_prefill_attn_ws_bytes(const Dims& d, int T);
hipError_t fast_prefill_attn(const Dims& d, const void* q, const void* k, const void* v, int T, void* o,
                             void* ws, hipStream_t s);

}  // namespace mla
