// C ABI of the MLA library: argument validation, workspace layout and kernel
// dispatch.  Nothing here synchronises the host or allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstdio>
#include <mutex>

#include "mla.h"
#include "mla_kernels.h"
#include "mla_fast.h"

using namespace mla;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Sequential carving of the caller's workspace into 256-byte aligned pieces.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + used) : nullptr;
    used += align_up(count * sizeof(T));
    return p;
  }
};

size_t act_bytes(const Dims& d) { return d.act == 0 ? 4 : 2; }

mla_status check_cfg(const mla_config* c, Dims* d) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->n_heads <= 0 || c->q_lora_rank < 0 || c->kv_lora_rank <= 0 || c->qk_nope <= 0 ||
      c->qk_rope <= 0 || c->v_dim <= 0 || c->block_size <= 0)
    return MLA_ERR_INVALID_ARG;
  if (c->qk_rope % 2 != 0) return MLA_ERR_INVALID_ARG;
  if (!(c->softmax_scale > 0.f) || !std::isfinite(c->softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (!(c->norm_eps >= 0.f) || !std::isfinite(c->norm_eps)) return MLA_ERR_INVALID_ARG;
  const bool ok_pair = (c->act_dtype == MLA_F32 && c->weight_dtype == MLA_F32) ||
                       (c->act_dtype == MLA_BF16 && c->weight_dtype == MLA_BF16) ||
                       (c->act_dtype == MLA_BF16 && c->weight_dtype == MLA_FP8_E4M3);
  if (!ok_pair) return MLA_ERR_UNSUPPORTED;
  // limits of the general kernels' per-thread arrays and LDS tiles
  if (c->kv_lora_rank > 1024 || c->qk_nope + c->qk_rope > 256 || c->v_dim > 256) return MLA_ERR_UNSUPPORTED;
  if (c->act_quant != 0 && c->act_quant != 1) return MLA_ERR_INVALID_ARG;
  if (c->act_quant == 1 && !(c->act_dtype == MLA_BF16 && c->weight_dtype == MLA_FP8_E4M3)) return MLA_ERR_UNSUPPORTED;
  d->D = c->hidden;
  d->H = c->n_heads;
  d->Lq = c->q_lora_rank;
  d->Lkv = c->kv_lora_rank;
  d->dn = c->qk_nope;
  d->dr = c->qk_rope;
  d->dv = c->v_dim;
  d->scale = c->softmax_scale;
  d->eps = c->norm_eps;
  d->bs = c->block_size;
  d->act = c->act_dtype == MLA_F32 ? 0 : 1;
  d->wk = c->weight_dtype == MLA_F32 ? W_F32 : (c->weight_dtype == MLA_BF16 ? W_BF16 : W_FP8);
  d->aq = c->act_quant;
  return MLA_OK;
}

bool check_weight(const Dims& d, const mla_weight& w) {
  if (!w.w) return false;
  if (d.wk == W_FP8) return w.scale != nullptr;
  return true;
}

WeightView view(const Dims& d, const mla_weight& w, int64_t N) {
  WeightView v;
  v.w = w.w;
  v.scale = w.scale;
  v.ld = N;
  v.scale_ld = (int)((N + 127) / 128);
  return v;
}

// ---- workspace layouts (the single source of truth for sizes and pointers) ----------
// Every projection result is kept as fp32 split-K partial sums (one part on the general
// path) and summed by the kernel that consumes it.
size_t proj_out_bytes(const Dims& d, int M, int N, int K) {
  if (fast_proj_supported(d)) return fast_gemm_out_bytes(d, M, N, K);
  return (size_t)M * N * sizeof(float);
}

// Quantised activations of one projection (act_quant): codes + exponents for the fp8 kernel,
// or dequantised bf16 rows for the other kernels.
size_t quant_bytes(const Dims& d, int M, int N, int K, int n_split) {
  if (!d.aq) return 0;
  if (fast_gemm_f8_ok(d, M, N, K, n_split)) {
    const size_t m_pad = (size_t)f8_rows_pad(M);
    return align_up((size_t)M * K) + align_up((size_t)((K + 127) / 128) * m_pad);
  }
  return align_up((size_t)M * K * 2);
}

// output columns of the stage-1 projection: [q latent (Lq) or query (H*dqk) | c_kv | k_pe]
int stage1_q_cols(const Dims& d) { return d.Lq > 0 ? d.Lq : d.H * d.dqk(); }

struct QkvWs {
  void* qz;    // quantised activations of the projection in flight (act_quant)
  void* xn;    // [n, D]                  x after the layer-input RMSNorm (act), when input_norm_w is given
  float* P1;   // [n, stage1_q_cols + R]  stage-1 projection
  float* P2;   // [n, H*dqk]              query up-projection (Lq > 0)
  void* cqn;   // [n, Lq]                 RMSNorm(q latent) * gamma (act)
  void* cn;    // [n, Lkv]                RMSNorm(c_kv) * gamma (act), prefill only
  float* PKV;  // [n, H*(dn+dv)]          kv up-projection, prefill only
};

size_t qkv_ws(const Dims& d, int n, bool prefill, void* base, QkvWs* out) {
  Carver c(base);
  QkvWs w;
  const int HQ = d.H * d.dqk();
  const int NKV = d.H * (d.dn + d.dv);
  size_t qz = quant_bytes(d, n, stage1_q_cols(d) + d.R(), d.D, stage1_q_cols(d));
  if (d.Lq > 0) qz = std::max(qz, quant_bytes(d, n, HQ, d.Lq, HQ));
  if (prefill) qz = std::max(qz, quant_bytes(d, n, NKV, d.Lkv, NKV));
  w.qz = c.take<char>(qz);
  w.xn = c.take<char>((size_t)n * d.D * act_bytes(d));
  w.P1 = (float*)c.take<char>(proj_out_bytes(d, n, stage1_q_cols(d) + d.R(), d.D));
  // results handed straight to their consumer need no buffer
  const bool q_fused = fast_gemm_fusable(d, n, HQ, d.Lq, HQ, GemmEpilogue::QUERY);
  const bool kv_fused = fast_gemm_fusable(d, n, NKV, d.Lkv, NKV, GemmEpilogue::KV);
  w.P2 = d.Lq > 0 ? (float*)c.take<char>(q_fused ? 0 : proj_out_bytes(d, n, HQ, d.Lq)) : nullptr;
  w.cqn = d.Lq > 0 ? c.take<char>((size_t)n * d.Lq * act_bytes(d)) : nullptr;
  w.cn = prefill ? c.take<char>((size_t)n * d.Lkv * act_bytes(d)) : nullptr;
  w.PKV = prefill ? (float*)c.take<char>(kv_fused ? 0 : proj_out_bytes(d, n, NKV, d.Lkv)) : nullptr;
  if (out) *out = w;
  return c.used;
}

struct DecodeAttnWs {
  float* Qabs;     // [B, H, R]
  float* part_o;   // [B*H*nsplit, Lkv]
  float* part_ml;  // [B*H*nsplit, 2]
  int nsplit, chunk;
  FastDecodeWs fast;
};

void decode_split_plan(int max_context, int* nsplit, int* chunk) {
  int ch = 1024;
  while ((max_context + ch - 1) / ch > 16) ch *= 2;
  *chunk = ch;
  *nsplit = (max_context + ch - 1) / ch;
  if (*nsplit < 1) *nsplit = 1;
}

size_t decode_attn_ws(const Dims& d, int B, int max_context, void* base, DecodeAttnWs* out) {
  Carver c(base);
  DecodeAttnWs w;
  if (fast_decode_supported(d)) {
    const size_t need = fast_decode_ws_bytes(d, B, max_context);
    w.fast.base = c.take<char>(need);
    w.fast.bytes = need;
    w.Qabs = nullptr;
    w.part_o = w.part_ml = nullptr;
    w.nsplit = w.chunk = 0;
  } else {
    decode_split_plan(max_context, &w.nsplit, &w.chunk);
    w.Qabs = c.take<float>((size_t)B * d.H * d.R());
    w.part_o = c.take<float>((size_t)B * d.H * w.nsplit * d.Lkv);
    w.part_ml = c.take<float>((size_t)B * d.H * w.nsplit * 2);
  }
  if (out) *out = w;
  return c.used;
}

// Chunked prefill over a paged prefix: the decode workspace for T queries plus their
// context lengths.
size_t chunk_attn_ws(const Dims& d, int T, int max_context, void* base, DecodeAttnWs* out, int32_t** ctx) {
  Carver c(base);
  const size_t dec = decode_attn_ws(d, T, max_context, base, out);
  c.used = align_up(dec);
  int32_t* p = c.take<int32_t>((size_t)T);
  if (ctx) *ctx = p;
  return c.used;
}

// Expanded chunk attention: rows 0 .. N-1 of the sequence gathered from the paged cache
// (latent parts, rope part of K), expanded by wkv_b into K (k_nope) and V.
struct ChunkExpWs {
  void* c;     // [N, Lkv]
  void* K;     // [N, H, dqk]
  void* V;     // [N, H, dv]
  float* PKV;  // [N, H*(dn+dv)] partials, when the expansion is not handed straight to K and V
};

size_t chunk_exp_ws(const Dims& d, int N, void* base, ChunkExpWs* out) {
  Carver c(base);
  ChunkExpWs w;
  const int NKV = d.H * (d.dn + d.dv);
  const bool fused = fast_gemm_fusable(d, N, NKV, d.Lkv, NKV, GemmEpilogue::KV);
  w.c = c.take<char>((size_t)N * d.Lkv * 2);
  w.K = c.take<char>((size_t)N * d.H * d.dqk() * 2);
  w.V = c.take<char>((size_t)N * d.H * d.dv * 2);
  w.PKV = (float*)c.take<char>(fused ? 0 : proj_out_bytes(d, N, NKV, d.Lkv));
  if (out) *out = w;
  return c.used;
}

// Whether T queries after `prefix` cached rows take the expanded form: 2*H*(dqk+dv) flop per
// (query, row) pair instead of the absorbed 2*H*(2*Lkv+dr), for 2*H*Lkv*(dn+dv) per row of
// expansion.  The advantage grows with prefix (for a fixed T), so the largest prefix decides
// whether any call of a given T and max_context can take it.
bool chunk_expanded(const Dims& d, int T, int prefix) {
  if (d.aq || d.act != 1 || !fast_prefill_attn_supported(d) || !fast_proj_supported(d) || d.Lkv % 8 || d.dr % 8 ||
      d.dn % 8)
    return false;
  const double N = (double)prefix + T, pairs = (double)T * prefix + (double)T * (T + 1) / 2;
  const double saved = 2.0 * (2 * d.Lkv + d.dr) - 2.0 * (d.dqk() + d.dv);
  return pairs * saved > N * 2.0 * d.Lkv * (d.dn + d.dv);
}

size_t chunk_ws_need(const Dims& d, int T, int max_context) {
  size_t need = chunk_attn_ws(d, T, max_context, nullptr, nullptr, nullptr);
  if (chunk_expanded(d, T, std::max(0, max_context - T)))
    need = std::max(need, chunk_exp_ws(d, std::max(max_context, T), nullptr, nullptr));
  return need;
}

size_t out_proj_ws(const Dims& d, int M, void* base, float** Y, void** qz = nullptr) {
  Carver c(base);
  const bool fused = fast_gemm_fusable(d, M, d.D, d.H * d.dv, d.D, GemmEpilogue::STORE);
  float* y = (float*)c.take<char>(fused ? 0 : proj_out_bytes(d, M, d.D, d.H * d.dv));
  void* q = c.take<char>(quant_bytes(d, M, d.D, d.H * d.dv, d.D));
  if (Y) *Y = y;
  if (qz) *qz = q;
  return c.used;
}

// Scratch of mla_decode_attn_absorbed_noalloc: file-scope device memory, one copy per GPU for
// the life of the process.  Host code never uses the symbol's name as an address; the address
// is looked up once per device (hipGetSymbolAddress with that device current) and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_MIB << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

mla_status hip_status(hipError_t e) {
  if (e != hipSuccess) {
    if (std::getenv("MLA_TRACE")) std::fprintf(stderr, "mla: HIP error %s\n", hipGetErrorString(e));
    return MLA_ERR_HIP;
  }
  return MLA_OK;
}

#define HIP_TRY(expr)                                     \
  do {                                                    \
    hipError_t e_ = (expr);                               \
    if (e_ != hipSuccess) return hip_status(e_);          \
  } while (0)

// C = A @ [W0 | W1] (W0: output columns [0, n_split)), left as partial sums in `out`, or
// handed straight to the consumer `epi` describes (then *fused is set and the caller skips
// its own consumer kernel).
mla_status project(const Dims& d, const void* A, int64_t lda, const WeightView& W0, int n_split, const WeightView& W1,
                   int M, int N, int K, float* out, Partials* res, hipStream_t s, const GemmEpilogue* epi = nullptr,
                   bool* fused = nullptr, void* qz = nullptr) {
  if (fused) *fused = false;
  if (d.aq) {
    // MX fp8 activations: the fp8 matrix-core kernel when the shape allows, otherwise the same
    // quantised values, dequantised exactly to bf16, through the usual kernels
    if (fast_gemm_f8_ok(d, M, N, K, n_split)) {
      uint8_t* codes = (uint8_t*)qz;
      uint8_t* exps = codes + align_up((size_t)M * K);
      HIP_TRY(quant_mx((const bf16_t*)A, lda, M, K, codes, exps, true, nullptr, s));
      HIP_TRY(fast_gemm_f8(d, codes, exps, W0, n_split, W1, M, N, K, out, res, epi, fused, s));
      return MLA_OK;
    }
    HIP_TRY(quant_mx((const bf16_t*)A, lda, M, K, nullptr, nullptr, false, (bf16_t*)qz, s));
    A = qz;
    lda = K;
  }
  if (fast_proj_supported(d)) {
    HIP_TRY(fast_gemm(d, A, lda, W0, n_split, W1, M, N, K, out, res, epi, fused, s));
    return MLA_OK;
  }
  const int n0 = std::min(n_split, N);
  HIP_TRY(gemm_simt(d, A, lda, W0, out, N, M, n0, K, s));
  if (n0 < N) HIP_TRY(gemm_simt(d, A, lda, W1, out + n0, N, M, N - n0, K, s));
  *res = Partials{out, 1, 0, N};
  return MLA_OK;
}

// Shared front end of prefill and decode: the layer-input RMSNorm when its gamma is
// given, one projection of x by [wq_a | wkv_a] (by
// [wq_b | wkv_a] without a query latent), row builder, query up-projection and RoPE.
mla_status front_end(const Dims& d, const mla_weights* w, const void* x, int n, const float* cosT,
                     const float* sinT, void* q, void* kbuf, void* kv_cache, int64_t n_blocks,
                     const int32_t* slot_mapping, const QkvWs& ws, hipStream_t s) {
  const int64_t n_slots = kv_cache ? n_blocks * d.bs : 0;
  const int HQ = d.H * d.dqk();
  const int NQ1 = stage1_q_cols(d);
  if (w->input_norm_w) {
    HIP_TRY(input_norm(d, x, n, w->input_norm_w, ws.xn, s));
    x = ws.xn;
  }
  Partials P1;
  const WeightView w1q = d.Lq > 0 ? view(d, w->wq_a, d.Lq) : view(d, w->wq_b, HQ);
  // without a query latent the stage-1 projection holds the query itself: its RoPE may run in
  // the projection (the other columns stay partial sums for the row builder)
  GemmEpilogue e1;
  e1.kind = GemmEpilogue::QUERY;
  e1.seg1_partials = true;
  e1.y = q;
  e1.cosT = cosT;
  e1.sinT = sinT;
  bool q_done = false;
  mla_status st = project(d, x, d.D, w1q, NQ1, view(d, w->wkv_a, d.R()), n, NQ1 + d.R(), d.D, ws.P1, &P1, s,
                          d.Lq > 0 ? nullptr : &e1, &q_done, ws.qz);
  if (st != MLA_OK) return st;
  HIP_TRY(row_builder(d, P1, P1.offset(NQ1), n, w->q_norm_w, w->kv_norm_w, cosT, sinT, ws.cqn, ws.cn, kv_cache,
                      n_slots, slot_mapping, kbuf, s));
  Partials PQ = P1;
  if (d.Lq > 0) {
    const WeightView wqb = view(d, w->wq_b, HQ);
    GemmEpilogue epi;
    epi.kind = GemmEpilogue::QUERY;
    epi.y = q;
    epi.cosT = cosT;
    epi.sinT = sinT;
    bool fused = false;
    st = project(d, ws.cqn, d.Lq, wqb, HQ, wqb, n, HQ, d.Lq, ws.P2, &PQ, s, &epi, &fused, ws.qz);
    if (st != MLA_OK) return st;
    if (fused) return MLA_OK;
  }
  if (q_done) return MLA_OK;
  HIP_TRY(q_epilogue(d, PQ, n, cosT, sinT, q, s));
  return MLA_OK;
}

bool check_weights_front(const Dims& d, const mla_weights* w) {
  if (!w) return false;
  if (d.Lq > 0 && (!check_weight(d, w->wq_a) || !w->q_norm_w)) return false;
  return check_weight(d, w->wq_b) && check_weight(d, w->wkv_a) && w->kv_norm_w != nullptr;
}

// Shared by mla_decode_attn_absorbed and its no-alloc variant: validation, then the launches on
// the given workspace, or on the static scratch when use_scratch is set (ws and ws_bytes ignored).
mla_status decode_attn_entry(const mla_config* cfg, const mla_weights* w, const void* q, int32_t B,
                             const void* kv_cache, int64_t n_blocks, const int32_t* block_table, int32_t max_blocks,
                             const int32_t* context_lens, void* o, void* ws, size_t ws_bytes, bool use_scratch,
                             void* stream) {
  Dims d;
  mla_status st = check_cfg(cfg, &d);
  if (st != MLA_OK) return st;
  if (B <= 0 || !w || !q || !kv_cache || n_blocks <= 0 || !block_table || max_blocks <= 0 || !context_lens ||
      !o || !check_weight(d, w->wkv_b))
    return MLA_ERR_INVALID_ARG;
  const int64_t max_ctx64 = (int64_t)max_blocks * d.bs;
  if (max_ctx64 > (1 << 30)) return MLA_ERR_UNSUPPORTED;
  const int max_ctx = (int)max_ctx64;
  if (use_scratch) {
    if (decode_attn_ws(d, B, max_ctx, nullptr, nullptr) > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
    HIP_TRY(scratch_address(&ws));
    ws_bytes = kNoAllocScratchBytes;
  }
  DecodeAttnWs L;
  const size_t need = decode_attn_ws(d, B, max_ctx, ws, &L);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const WeightView wkv_b = view(d, w->wkv_b, (int64_t)d.H * (d.dn + d.dv));
  if (fast_decode_supported(d)) {
    HIP_TRY(fast_decode_attn(d, q, B, kv_cache, n_blocks, block_table, max_blocks, max_blocks, context_lens,
                             wkv_b, o, L.fast, s));
    return MLA_OK;
  }
  HIP_TRY(fold_simt(d, q, B, wkv_b, L.Qabs, s));
  HIP_TRY(decode_attn_simt(d, L.Qabs, B, kv_cache, n_blocks, block_table, max_blocks, max_blocks, context_lens,
                           L.nsplit, L.chunk, L.part_o, L.part_ml, s));
  HIP_TRY(combine_simt(d, B, L.nsplit, L.part_o, L.part_ml, wkv_b, o, s));
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dtype combination or shape";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t mla_workspace_size(const mla_config* cfg, int32_t fn, int32_t n, int32_t max_context) {
  Dims d;
  if (check_cfg(cfg, &d) != MLA_OK || n <= 0) return 0;
  switch (fn) {
    case MLA_FN_QKV_PREFILL: return qkv_ws(d, n, true, nullptr, nullptr);
    case MLA_FN_PREFILL_ATTN: return fast_prefill_attn_ws_bytes(d, n);
    case MLA_FN_DECODE_QKV: return qkv_ws(d, n, false, nullptr, nullptr);
    case MLA_FN_DECODE_ATTN:
      if (max_context <= 0) return 0;
      return decode_attn_ws(d, n, max_context, nullptr, nullptr);
    case MLA_FN_OUT_PROJ: return out_proj_ws(d, n, nullptr, nullptr);
    case MLA_FN_PREFILL_ATTN_PAGED:
      if (max_context <= 0) return 0;
      return chunk_ws_need(d, n, max_context);
  }
  return 0;
}

mla_status mla_quantize_fp8(const void* x, int32_t M, int32_t K, int64_t ldx, uint8_t* codes, uint8_t* exps,
                            void* stream) {
  if (!x || !codes || !exps || M <= 0 || K <= 0 || ldx < K) return MLA_ERR_INVALID_ARG;
  HIP_TRY(quant_mx((const bf16_t*)x, ldx, M, K, codes, exps, false, nullptr, (hipStream_t)stream));
  return MLA_OK;
}

mla_status mla_rope_inv_freq(const mla_rope* r, int32_t qk_rope, double* inv_freq, void* stream) {
  if (!r || !inv_freq || qk_rope <= 0 || qk_rope % 2 != 0) return MLA_ERR_INVALID_ARG;
  if (!(r->theta > 1.0) || !std::isfinite(r->theta) || std::isnan(r->factor)) return MLA_ERR_INVALID_ARG;
  if (r->factor > 1.0 && (!std::isfinite(r->factor) || r->original_max_position <= 0 || !(r->beta_slow > 0.0) ||
                          !(r->beta_fast > r->beta_slow) || !std::isfinite(r->beta_fast)))
    return MLA_ERR_INVALID_ARG;
  HIP_TRY(rope_inv_freq(qk_rope, r->theta, r->factor, r->original_max_position, r->beta_fast, r->beta_slow,
                        inv_freq, (hipStream_t)stream));
  return MLA_OK;
}

double mla_rope_score_scale(const mla_rope* r, int32_t qk_nope, int32_t qk_rope) {
  if (qk_nope < 0 || qk_rope <= 0) return 0.0;
  double m = 1.0;
  if (r && r->factor > 1.0) m = 0.1 * r->mscale_all_dim * std::log(r->factor) + 1.0;
  return m * m / std::sqrt((double)qk_nope + (double)qk_rope);
}

mla_status mla_rope_tables(int32_t n, int32_t qk_rope, const int32_t* positions, int32_t pos_offset,
                           const double* inv_freq, float* cos, float* sin, void* stream) {
  if (n <= 0 || qk_rope <= 0 || qk_rope % 2 != 0 || !cos || !sin) return MLA_ERR_INVALID_ARG;
  HIP_TRY(rope_tables(n, qk_rope, positions, pos_offset, inv_freq, cos, sin, (hipStream_t)stream));
  return MLA_OK;
}

mla_status mla_qkv_prefill(const mla_config* cfg, const mla_weights* w, const void* x, int32_t T,
                           const float* cos, const float* sin, void* q, void* k, void* v,
                           void* kv_cache, const int32_t* slot_mapping, int64_t n_blocks,
                           void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  mla_status st = check_cfg(cfg, &d);
  if (st != MLA_OK) return st;
  if (T <= 0 || !x || !cos || !sin || !q || ((k == nullptr) != (v == nullptr)) || !check_weights_front(d, w) ||
      (k && !check_weight(d, w->wkv_b)))
    return MLA_ERR_INVALID_ARG;
  if ((kv_cache == nullptr) != (slot_mapping == nullptr)) return MLA_ERR_INVALID_ARG;
  if (kv_cache && n_blocks <= 0) return MLA_ERR_INVALID_ARG;
  QkvWs L;
  const size_t need = qkv_ws(d, T, true, ws, &L);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  st = front_end(d, w, x, T, cos, sin, q, k, kv_cache, n_blocks, slot_mapping, L, s);
  if (st != MLA_OK || !k) return st;
  const int NKV = d.H * (d.dn + d.dv);
  const WeightView wkvb = view(d, w->wkv_b, NKV);
  Partials PKV;
  GemmEpilogue epi;
  epi.kind = GemmEpilogue::KV;
  epi.y = k;
  epi.y2 = v;
  bool fused = false;
  st = project(d, L.cn, d.Lkv, wkvb, NKV, wkvb, T, NKV, d.Lkv, L.PKV, &PKV, s, &epi, &fused, L.qz);
  if (st != MLA_OK) return st;
  if (!fused) HIP_TRY(kv_split(d, PKV, T, k, v, s));
  return MLA_OK;
}

mla_status mla_prefill_attn(const mla_config* cfg, const void* q, const void* k, const void* v, int32_t T,
                            void* o, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  mla_status st = check_cfg(cfg, &d);
  if (st != MLA_OK) return st;
  if (T <= 0 || !q || !k || !v || !o) return MLA_ERR_INVALID_ARG;
  const size_t need = fast_prefill_attn_ws_bytes(d, T);
  if (need > 0 && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (fast_prefill_attn_supported(d))
    HIP_TRY(fast_prefill_attn(d, q, k, v, T, o, ws, s));
  else
    HIP_TRY(prefill_attn_simt(d, q, k, v, T, o, s));
  return MLA_OK;
}

mla_status mla_decode_qkv_and_scatter(const mla_config* cfg, const mla_weights* w, const void* x,
                                      int32_t B, const float* cos, const float* sin, void* kv_cache,
                                      int64_t n_blocks, const int32_t* slot_mapping, void* q,
                                      void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  mla_status st = check_cfg(cfg, &d);
  if (st != MLA_OK) return st;
  if (B <= 0 || !x || !cos || !sin || !q || !kv_cache || !slot_mapping || n_blocks <= 0 ||
      !check_weights_front(d, w))
    return MLA_ERR_INVALID_ARG;
  QkvWs L;
  const size_t need = qkv_ws(d, B, false, ws, &L);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  return front_end(d, w, x, B, cos, sin, q, nullptr, kv_cache, n_blocks, slot_mapping, L, (hipStream_t)stream);
}

mla_status mla_decode_attn_absorbed(const mla_config* cfg, const mla_weights* w, const void* q,
                                    int32_t B, const void* kv_cache, int64_t n_blocks,
                                    const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* context_lens, void* o, void* ws,
                                    size_t ws_bytes, void* stream) {
  return decode_attn_entry(cfg, w, q, B, kv_cache, n_blocks, block_table, max_blocks, context_lens, o, ws, ws_bytes,
                           false, stream);
}

mla_status mla_decode_attn_absorbed_noalloc(const mla_config* cfg, const mla_weights* w, const void* q, int32_t B,
                                            const void* kv_cache, int64_t n_blocks, const int32_t* block_table,
                                            int32_t max_blocks, const int32_t* context_lens, void* o, void* stream) {
  return decode_attn_entry(cfg, w, q, B, kv_cache, n_blocks, block_table, max_blocks, context_lens, o, nullptr, 0,
                           true, stream);
}

mla_status mla_prefill_attn_paged(const mla_config* cfg, const mla_weights* w, const void* q, int32_t T,
                                  const void* kv_cache, int64_t n_blocks, const int32_t* block_table,
                                  int32_t max_blocks, int32_t prefix_len, void* o, void* ws, size_t ws_bytes,
                                  void* stream) {
  Dims d;
  mla_status st = check_cfg(cfg, &d);
  if (st != MLA_OK) return st;
  if (T <= 0 || prefix_len < 0 || !w || !q || !kv_cache || n_blocks <= 0 || !block_table || max_blocks <= 0 ||
      !o || !check_weight(d, w->wkv_b))
    return MLA_ERR_INVALID_ARG;
  const int64_t max_ctx64 = (int64_t)max_blocks * d.bs;
  if ((int64_t)prefix_len + T > max_ctx64) return MLA_ERR_INVALID_ARG;
  if (max_ctx64 > (1 << 30)) return MLA_ERR_UNSUPPORTED;
  const int max_ctx = (int)max_ctx64;
  hipStream_t s = (hipStream_t)stream;
  const int NKV = d.H * (d.dn + d.dv);
  const WeightView wkv_b = view(d, w->wkv_b, NKV);
  if (chunk_expanded(d, T, prefix_len)) {
    // rows 0 .. N-1 expanded to per-head keys and values, then causal attention with the
    // queries at positions prefix_len ..
    const int N = prefix_len + T;
    ChunkExpWs E;
    const size_t need = chunk_exp_ws(d, N, ws, &E);
    if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
    HIP_TRY(chunk_gather(d, kv_cache, n_blocks, block_table, N, E.c, E.K, s));
    Partials PKV;
    GemmEpilogue epi;
    epi.kind = GemmEpilogue::KV;
    epi.y = E.K;
    epi.y2 = E.V;
    bool fused = false;
    st = project(d, E.c, d.Lkv, wkv_b, NKV, wkv_b, N, NKV, d.Lkv, E.PKV, &PKV, s, &epi, &fused, nullptr);
    if (st != MLA_OK) return st;
    if (!fused) HIP_TRY(kv_split(d, PKV, N, E.K, E.V, s));
    HIP_TRY(fast_prefill_attn_offset(d, q, E.K, E.V, T, prefix_len, o, nullptr, s));
    return MLA_OK;
  }
  DecodeAttnWs L;
  int32_t* ctx = nullptr;
  const size_t need = chunk_attn_ws(d, T, max_ctx, ws, &L, &ctx);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  HIP_TRY(chunk_ctx(T, prefix_len, ctx, s));
  // every query of the chunk is a decode query of the same sequence at its own position:
  // one block-table row shared by all (stride 0) and context length prefix + t + 1
  if (fast_decode_supported(d)) {
    HIP_TRY(fast_decode_attn(d, q, T, kv_cache, n_blocks, block_table, max_blocks, 0, ctx, wkv_b, o, L.fast, s));
    return MLA_OK;
  }
  HIP_TRY(fold_simt(d, q, T, wkv_b, L.Qabs, s));
  HIP_TRY(decode_attn_simt(d, L.Qabs, T, kv_cache, n_blocks, block_table, max_blocks, 0, ctx, L.nsplit, L.chunk,
                           L.part_o, L.part_ml, s));
  HIP_TRY(combine_simt(d, T, L.nsplit, L.part_o, L.part_ml, wkv_b, o, s));
  return MLA_OK;
}

mla_status mla_out_proj(const mla_config* cfg, const mla_weights* w, const void* o, int32_t M, void* y,
                        void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  mla_status st = check_cfg(cfg, &d);
  if (st != MLA_OK) return st;
  if (M <= 0 || !w || !o || !y || !check_weight(d, w->wo)) return MLA_ERR_INVALID_ARG;
  float* Y = nullptr;
  void* qz = nullptr;
  const size_t need = out_proj_ws(d, M, ws, &Y, &qz);
  if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int K = d.H * d.dv;
  const WeightView wo = view(d, w->wo, d.D);
  Partials P;
  GemmEpilogue epi;
  epi.kind = GemmEpilogue::STORE;
  epi.y = y;
  bool fused = false;
  st = project(d, o, K, wo, d.D, wo, M, d.D, K, Y, &P, s, &epi, &fused, qz);
  if (st != MLA_OK) return st;
  if (!fused) HIP_TRY(cast_rows(d, P, M, d.D, y, s));
  return MLA_OK;
}

}  // extern "C"
