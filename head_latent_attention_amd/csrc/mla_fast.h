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

// Consumers a projection can hand its result to directly when K is not split:
//   STORE  y[m, n] = C[m, n] (act)
//   QUERY  q[m, h, :] = [C[m, h*dqk : +dn] | RoPE_m(C[m, h*dqk+dn : (h+1)*dqk])] (act)
//   KV     k[m, h, j] = C[m, h*(dn+dv) + j] (j < dn), v[m, h, j - dn] = the rest (act)
struct GemmEpilogue {
  enum Kind { PARTIALS = 0, STORE = 1, QUERY = 2, KV = 3 };
  int kind = PARTIALS;
  // the consumer takes W0's columns [0, n_split) only (y with row stride n_split); W1's columns
  // stay partial sums in `out` (QUERY on the large-tile path: the query RoPE of a projection
  // without a query latent, whose other columns feed the row builder)
  bool seg1_partials = false;
  void* y = nullptr;   // STORE: y; QUERY: q; KV: k
  void* y2 = nullptr;  // KV: v
  const float* cosT = nullptr;
  const float* sinT = nullptr;
};

// Projection GEMM / GEMV: C[M, N] = A[M, K] (act) @ [W0 | W1], W0 giving output columns
// [0, n_split) and W1 columns [n_split, N) (n_split >= N: W0 only).  C is left in `out`
// (fast_gemm_out_bytes(M, N, K) bytes) as split-K partial sums, described by *res; or, when
// `epi` asks for a consumer and K is not split, written straight to it (*fused = true).
bool fast_proj_supported(const Dims& d);
size_t fast_gemm_out_bytes(const Dims& d, int M, int N, int K);
// whether fast_gemm hands the result of this shape straight to a consumer of `kind`
bool fast_gemm_fusable(const Dims& d, int M, int N, int K, int n_split, int kind);
hipError_t fast_gemm(const Dims& d, const void* A, int64_t lda, const WeightView& W0, int n_split,
                     const WeightView& W1, int M, int N, int K, float* out, Partials* res,
                     const GemmEpilogue* epi, bool* fused, hipStream_t s);

// Compute units of the current device (cached per device); persistent kernels size their
// grids with it.  Any positive grid is correct for them, so a failed query returns 256.
int device_cu_count();

// Absorbed decode: fold, split-context attention over the paged cache, combine with W_UV.
bool fast_decode_supported(const Dims& d);
size_t fast_decode_ws_bytes(const Dims& d, int B, int max_context);
// Query b reads its block ids from block_table + b * bt_stride (0: one shared table).
hipError_t fast_decode_attn(const Dims& d, const void* q, int B, const void* cache, int64_t n_blocks,
                            const int32_t* block_table, int max_blocks, int64_t bt_stride, const int32_t* ctx,
                            const WeightView& wkv_b, void* o, const FastDecodeWs& ws, hipStream_t s);

// fp8 projection for M > 1024 with quantised activations: A8 E4M3FN codes [M, K] (row stride
// K), Ae E8M0 exponents (one power-of-two scale per row and 128 columns) [K/128][f8_rows_pad(M)]
// in f8_exp_order, fp8
// weights whose block scales are powers of two (others make the outputs NaN).  Same result
// hand-over as fast_gemm.  fast_gemm_f8_ok tells whether the shape is supported.
bool fast_gemm_f8_ok(const Dims& d, int M, int N, int K, int n_split);
// Rows of the exponent array: M padded to the fp8 kernel's 256-row tile, so that every row a
// tile addresses has a byte.
__host__ __device__ __forceinline__ int64_t f8_rows_pad(int64_t M) { return (M + 255) / 256 * 256; }
// Byte index of the exponent of row m, 128-column group kg, rows padded to m_pad
// (f8_rows_pad): per group, per block of 128 rows, row 16 mt + j at 8 j + mt.
__host__ __device__ __forceinline__ int64_t f8_exp_order(int64_t kg, int64_t m, int64_t m_pad) {
  const int64_t r = m & 127;
  return kg * m_pad + (m - r) + 8 * (r & 15) + (r >> 4);
}
hipError_t fast_gemm_f8(const Dims& d, const uint8_t* A8, const uint8_t* Ae, const WeightView& W0, int n_split,
                        const WeightView& W1, int M, int N, int K, float* out, Partials* res,
                        const GemmEpilogue* epi, bool* fused, hipStream_t s);

// Causal prefill flash attention.
bool fast_prefill_attn_supported(const Dims& d);
size_t fast_prefill_attn_ws_bytes(const Dims& d, int T);
hipError_t fast_prefill_attn(const Dims& d, const void* q, const void* k, const void* v, int T, void* o,
                             void* ws, hipStream_t s);
// The same with query row t at position q_off + t: k and v hold q_off + T rows, and query t sees
// rows 0 .. q_off + t (a chunk of a sequence after q_off cached positions).
hipError_t fast_prefill_attn_offset(const Dims& d, const void* q, const void* k, const void* v, int T, int q_off,
                                    void* o, void* ws, hipStream_t s);

}  // namespace mla
