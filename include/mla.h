/*
 * mla.h -- C ABI of the MI355X (gfx950) multi-head latent attention (MLA) hot path.
 *
 * The layer is the DeepSeek-V2/V3 MLA described by:
 *   [NeMo-MLA]   NVIDIA NeMo AutoModel, nemo_automodel.components.models.deepseek_v3.layers, class MLA
 *   [Mla]        logicaffeine_compile, model::spec, Struct Mla
 *   [MlaWeights] atlas docs, spark_model::layers::qwen3_attention, Struct MlaWeights
 *   [NKI-Decode] AWS Neuron NKI, "MLA Decode QKV Kernel API Reference"
 *   [NKI-CTE]    AWS Neuron NKI, "QKV CTE MLA Kernel API Reference"
 *   [YaRN]       Peng et al., "YaRN: Efficient Context Window Extension of Large Language
 *                Models" (2023), the method behind the [Mla] scale and [MlaWeights] yarn_inv_freq
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller.  The library keeps
 *     no pointer after a call returns; buffers must stay alive until `stream`
 *     reaches the enqueued work.
 *   - Calls only enqueue work on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream).  They never synchronise the host, never copy device to
 *     host and never allocate device memory: scratch comes from the caller's
 *     workspace `ws` of `ws_bytes` bytes (see mla_workspace_size).  Workspace
 *     contents are undefined after a call.  Two calls that share a workspace must
 *     be ordered on one stream.
 *   - Tensors are dense row-major with the shapes given below.  "act" tensors
 *     (x, q, k, v, o, y and the latent cache) have cfg->act_dtype; weights have
 *     cfg->weight_dtype.  Supported (act, weight) pairs: (F32, F32), (BF16, BF16),
 *     (BF16, FP8_E4M3).
 *   - Dimension names: D = hidden, H = n_heads, Lq = q_lora_rank, Lkv = kv_lora_rank,
 *     dn = qk_nope, dr = qk_rope, dv = v_dim, dqk = dn + dr, R = Lkv + dr (the width
 *     of one latent-cache row), bs = block_size.
 *   - Arguments are validated on the host before anything is enqueued; a failed
 *     check returns a negative status and leaves every output untouched.  HIP
 *     launch failures return MLA_ERR_HIP.  No C++ exception crosses this ABI.
 *   - Paging indices (slot_mapping, block_table, context_lens) live on the device
 *     and are not inspected by the host.  Kernels skip a slot outside
 *     [0, n_blocks*bs) and treat a block id outside [0, n_blocks) as a row that
 *     contributes nothing, so bad indices give wrong numbers, never a memory fault.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,  /* null pointer, non-positive or odd dimension, bad count */
  MLA_ERR_UNSUPPORTED = -2,  /* dtype pair or shape the kernels do not implement      */
  MLA_ERR_WORKSPACE = -3,    /* ws_bytes smaller than mla_workspace_size(...)         */
  MLA_ERR_HIP = -4           /* a HIP launch or runtime call failed                   */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype;

/* The layer's parameters, after the logicaffeine Mla struct (fields heads,
 * q_lora_rank (optional), kv_lora_rank, qk_nope, qk_rope, v_dim, scale) and the
 * NKI decode-QKV kernel's scalar parameters (n_heads, qk_nope_head_dim,
 * qk_rope_head_dim, kv_lora_rank, norm_eps). */
typedef struct {
  int32_t hidden;         /* D                                                              */
  int32_t n_heads;        /* H                                                              */
  int32_t q_lora_rank;    /* Lq; 0 = no query latent, the query is x @ wq_b ([Mla] optional) */
  int32_t kv_lora_rank;   /* Lkv                                                            */
  int32_t qk_nope;        /* dn: per-head query/key dims that do not rotate                 */
  int32_t qk_rope;        /* dr: trailing per-head dims that rotate; must be even           */
  int32_t v_dim;          /* dv                                                             */
  float softmax_scale;    /* score scale, normally 1/sqrt(dn + dr) ([NeMo-MLA] softmax_scale) */
  float norm_eps;         /* RMSNorm epsilon, normally 1e-6 ([NKI-Decode] norm_eps)          */
  int32_t block_size;     /* bs: rows per paged-cache block                                 */
  int32_t act_dtype;      /* mla_dtype: MLA_F32 or MLA_BF16                                 */
  int32_t weight_dtype;   /* mla_dtype: MLA_F32, MLA_BF16 or MLA_FP8_E4M3                   */
  int32_t act_quant;      /* 0: activations enter the projections as act_dtype.  1 (BF16 act,
                             FP8_E4M3 weights only): every activation entering a projection
                             (x, the normed q and kv latents, o) is MX fp8-quantised as
                             mla_quantize_fp8 does, and large projections run on the fp8 matrix
                             cores ([NKI-CTE] qkv_mla_mx: MX fp8 with 8-bit power-of-two scales).
                             The weight block scales must then be powers of two (the compact
                             scales of [NKI-CTE]); a projection of M > 1024 rows gives NaN
                             outputs for a block whose scale is not.                        */
} mla_config;

/* One projection weight [K, N] row-major ("in, out" orientation, as the NKI
 * kernels take wq_a [hidden, q_lora_rank] and wkv_a [hidden, kv_row_dim]).
 * For MLA_FP8_E4M3, `w` holds one OCP E4M3FN byte per element and `scale` is
 * fp32 [ceil(K/128), ceil(N/128)]: element (k, n) is code(k, n) * scale[k/128][n/128]
 * (the 128x128 block scales of the [MlaWeights] fp8 fields).  Otherwise scale is NULL. */
typedef struct {
  const void* w;
  const float* scale;
} mla_weight;

typedef struct {
  mla_weight wq_a;   /* [D, Lq] query down-projection; unused when Lq == 0                     */
  mla_weight wq_b;   /* [Lq, H*dqk] (or [D, H*dqk] when Lq == 0); per head [q_nope | q_pe]     */
  mla_weight wkv_a;  /* [D, R] -> one cache row [c_kv | k_pe] per token                        */
  mla_weight wkv_b;  /* [Lkv, H*(dn+dv)]; per head [k_nope | v].  Its per-head column blocks
                        are the absorption weights W_UK (first dn) and W_UV (last dv)          */
  mla_weight wo;     /* [H*dv, D] output projection                                            */
  const float* q_norm_w;   /* [Lq]  fp32 RMSNorm gamma of the query latent; unused when Lq == 0 */
  const float* kv_norm_w;  /* [Lkv] fp32 RMSNorm gamma of the KV latent                         */
  const float* input_norm_w;  /* [D] fp32 gamma of the layer's input RMSNorm, or NULL.  When given,
                                 the projection entry points normalise each row of x first:
                                 x * rsqrt(mean(x^2) + norm_eps) * input_norm_w ([NKI-Decode]
                                 input_norm_w: the input norm folded into the hidden load)      */
} mla_weights;

/* MX fp8 quantisation of bf16 rows, the form mla_config.act_quant applies to projection
 * inputs ([NKI-CTE] qkv_mla_mx: MX fp8 activations, 8-bit power-of-two scales).  For row m and
 * each group of 128 columns (the last may be shorter): e = the smallest integer with
 * max|x| <= 448 * 2^e (e = 0 for an all-zero group; clamped to [-127, 127]), and each element's
 * code is the OCP E4M3FN value nearest to x * 2^-e, ties to even.
 *   x      bf16 [M, K] device, row stride ldx >= K elements.
 *   codes  uint8 [M, K] device out (row stride K).
 *   exps   uint8 [ceil(K/128), M] device out: e + 127 (an E8M0 byte).
 * M, K >= 1. */
mla_status mla_quantize_fp8(const void* x, int32_t M, int32_t K, int64_t ldx, uint8_t* codes, uint8_t* exps,
                            void* stream);

/* Rotary-embedding frequencies ([MlaWeights] yarn_inv_freq / main_inv_freq; [Mla] scale).
 * Pair i of the qk_rope rotating dims turns by position * inv_freq[i] radians. */
typedef struct {
  double theta;                  /* base of the plain frequencies theta^(-2i/dr), normally 10000       */
  double factor;                 /* YaRN context-extension factor; <= 1 means plain RoPE                */
  int32_t original_max_position; /* context length the plain frequencies were trained for (factor > 1) */
  double beta_fast, beta_slow;   /* turn counts over that context bounding the blend (normally 32, 1)  */
  double mscale_all_dim;         /* m of YaRN's magnitude 0.1 * m * ln(factor) + 1 (normally 1)         */
} mla_rope;

/* Inverse frequencies inv_freq [qk_rope/2] (fp64, device, out).  factor <= 1: theta^(-2i/dr).
 * factor > 1, YaRN by parts ([YaRN] section 3.2): a pair whose wavelength 2*pi/f turns at least
 * beta_fast times over original_max_position keeps f; one that turns at most beta_slow times
 * gets f / factor; in between the share of f / factor grows linearly in the pair index from
 * floor(index where the count is beta_fast) (at least 0) to ceil(index where it is beta_slow)
 * (at most qk_rope - 1).  Requires theta > 1, qk_rope even; with factor > 1 also
 * original_max_position > 0 and beta_fast > beta_slow > 0. */
mla_status mla_rope_inv_freq(const mla_rope* rope, int32_t qk_rope, double* inv_freq, void* stream);

/* The score scale 1/sqrt(qk_nope + qk_rope) times the square of YaRN's magnitude
 * 0.1 * mscale_all_dim * ln(factor) + 1 (magnitude 1 when factor <= 1 or rope is NULL)
 * ([Mla] scale field; [YaRN] section 3.4).  Host-only; returns 0 for non-positive dims. */
double mla_rope_score_scale(const mla_rope* rope, int32_t qk_nope, int32_t qk_rope);

/* cos/sin tables for the projection entry points: for token t < n and pair i < qk_rope/2,
 *   angle = (positions[t] + pos_offset) * inv_freq[i],  cos[t][i] = cos(angle), sin[t][i] = sin(angle)
 * with the angle and its reduction to a quadrant (|remainder| <= pi/4) evaluated in fp64 and
 * cos/sin of the remainder in fp32 (results within about 1e-7 of the exact values).
 *   positions  int32 [n] device, or NULL for positions 0..n-1 (e.g. context_lens with
 *              pos_offset -1 gives each decode token's position).
 *   inv_freq   fp64 [qk_rope/2] device (mla_rope_inv_freq), or NULL for theta = 10000.
 *   cos, sin   fp32 [n, qk_rope/2] device out.
 * n >= 1, qk_rope even. */
mla_status mla_rope_tables(int32_t n, int32_t qk_rope, const int32_t* positions, int32_t pos_offset,
                           const double* inv_freq, float* cos, float* sin, void* stream);

/* Identifiers of the entry points, for mla_workspace_size. */
enum {
  MLA_FN_QKV_PREFILL = 0,
  MLA_FN_PREFILL_ATTN = 1,
  MLA_FN_DECODE_QKV = 2,
  MLA_FN_DECODE_ATTN = 3,
  MLA_FN_OUT_PROJ = 4,
  MLA_FN_PREFILL_ATTN_PAGED = 5
};

/* Context-encoding projections for T tokens at positions 0..T-1 of one sequence
 * ([NKI-CTE] qkv_mla_mx, Notes: stage 1 x @ [wq_a | wkv_a], split, RMSNorm of both
 * latents, stage 2 projections, final assembly).
 *   x     [T, D] act.
 *   cos, sin  fp32 [T, dr/2]: cos/sin of the angle of rope pair i at token t
 *         ([NKI-Decode] cos/sin parameters).  Pair (2i, 2i+1) rotates as a complex number.
 *   q     [T, H, dqk] act out: per head [q_nope | RoPE(q_pe)].
 *   k     [T, H, dqk] act out: per head [k_nope | RoPE(k_pe)], the rope key shared by all heads.
 *   v     [T, H, dv]  act out.
 *   kv_cache  [n_blocks, 1, bs, R] act, updated in place: row t = [RMSNorm(c_kv) | RoPE(k_pe)]
 *         is written to flat row slot_mapping[t] (block slot/bs, offset slot%bs); -1 skips.
 *         kv_cache and slot_mapping may both be NULL (no cache write).
 *   slot_mapping  int32 [T] or NULL.
 * k and v may both be NULL: the per-head expansion through wkv_b is skipped (wkv_b may then
 * be unset), as for a chunk whose attention runs on the latent cache (mla_prefill_attn_paged).
 * The cos/sin rows give the tokens' positions, so a chunk later in a sequence passes the
 * tables of its own positions.
 * T >= 1. */
mla_status mla_qkv_prefill(const mla_config* cfg, const mla_weights* w, const void* x, int32_t T,
                           const float* cos, const float* sin, void* q, void* k, void* v,
                           void* kv_cache, const int32_t* slot_mapping, int64_t n_blocks,
                           void* ws, size_t ws_bytes, void* stream);

/* Causal softmax attention of one sequence's T tokens, per head:
 *   o[t, h] = sum_{j <= t} softmax_j(scale * q[t,h] . k[j,h]) v[j,h]
 * ([NeMo-MLA] forward with a causal attention_mask and softmax_scale).
 *   q, k [T, H, dqk] act; v [T, H, dv] act; o [T, H, dv] act out.  T >= 1. */
mla_status mla_prefill_attn(const mla_config* cfg, const void* q, const void* k, const void* v,
                            int32_t T, void* o, void* ws, size_t ws_bytes, void* stream);

/* Decode front end for B sequences, one new token each ([NKI-Decode] mla_decode_qkv:
 * both projections, both RMSNorms, interleaved RoPE, and the scatter of this step's
 * row into the paged cache).  The query absorption that kernel also performs is done
 * by mla_decode_attn_absorbed here.
 *   x     [B, D] act.
 *   cos, sin  fp32 [B, dr/2] at each token's position.
 *   kv_cache  [n_blocks, 1, bs, R] act, updated: row b goes to flat row slot_mapping[b] (-1 skips).
 *   slot_mapping  int32 [B].
 *   q     [B, H, dqk] act out: per head [q_nope | RoPE(q_pe)] (not yet absorbed).
 * B >= 1. */
mla_status mla_decode_qkv_and_scatter(const mla_config* cfg, const mla_weights* w, const void* x,
                                      int32_t B, const float* cos, const float* sin, void* kv_cache,
                                      int64_t n_blocks, const int32_t* slot_mapping, void* q,
                                      void* ws, size_t ws_bytes, void* stream);

/* Absorbed decode attention over the paged latent cache ([NKI-Decode] background:
 * the query is absorbed into the cache's latent space; [MlaWeights] w_uk_t / w_uv).
 *   q_lat[b,h]  = q_nope[b,h] @ W_UK[h]    (W_UK[h][p][c] = wkv_b[c][h*(dn+dv) + p])
 *   s[b,h,t]    = scale * (q_lat[b,h] . c_t + q_pe[b,h] . k_pe_t),   t < context_lens[b]
 *   o[b,h]      = (sum_t softmax_t(s) c_t) @ W_UV[h]   (W_UV[h][c][j] = wkv_b[c][h*(dn+dv) + dn + j])
 * where row t = [c_t | k_pe_t] of sequence b lives in block block_table[b][t/bs] at offset t%bs.
 *   q        [B, H, dqk] act (as produced by mla_decode_qkv_and_scatter).
 *   kv_cache [n_blocks, 1, bs, R] act (read only).
 *   block_table  int32 [B, max_blocks]; entries past ceil(ctx/bs) are ignored.
 *   context_lens int32 [B], each in [1, max_blocks*bs]; it counts the current token,
 *                whose row must already be in the cache.
 *   o        [B, H, dv] act out.
 * B >= 1, max_blocks >= 1. */
mla_status mla_decode_attn_absorbed(const mla_config* cfg, const mla_weights* w, const void* q,
                                    int32_t B, const void* kv_cache, int64_t n_blocks,
                                    const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* context_lens, void* o, void* ws,
                                    size_t ws_bytes, void* stream);

/* mla_decode_attn_absorbed for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments (minus ws / ws_bytes), same kernels and the same results bit for bit.  Scratch comes
 * from a static device array of MLA_NOALLOC_SCRATCH_MIB MiB that the library holds on every GPU it
 * runs on until the process ends; no call allocates or frees anything.  A call whose workspace
 * need, mla_workspace_size(cfg, MLA_FN_DECODE_ATTN, B, max_blocks * block_size), exceeds that
 * capacity returns MLA_ERR_WORKSPACE before any launch (at the V3 shape, 128 heads, the limit is
 * B <= 119, for any context length).  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and give wrong results;
 * calls ordered on one stream are safe.  Nothing in the array has to start at any value: every
 * byte a call reads was written earlier in the same call. */
#define MLA_NOALLOC_SCRATCH_MIB 64
mla_status mla_decode_attn_absorbed_noalloc(const mla_config* cfg, const mla_weights* w, const void* q,
                                            int32_t B, const void* kv_cache, int64_t n_blocks,
                                            const int32_t* block_table, int32_t max_blocks,
                                            const int32_t* context_lens, void* o, void* stream);

/* Chunked prefill over a paged prefix: causal attention of T new tokens of one sequence over
 * that sequence's latent cache ([NKI-Decode] paged kv_cache).  Query t sits at position
 * prefix_len + t and attends to rows 0 .. prefix_len + t, read through block_table.  Two forms
 * compute the same attention; the cheaper one is taken:
 *   absorbed ([MlaWeights] w_uk_block_diag / w_uv_block_diag: query absorption and value
 *     extraction used for prefill too): each query as mla_decode_attn_absorbed computes a decode
 *     query with context prefix_len + t + 1;
 *   expanded (bf16 activations without act_quant, V2/V3 head shape): the sequence's rows are
 *     expanded by wkv_b into per-head keys and values once, then causal attention as
 *     mla_prefill_attn with the queries offset by prefix_len.  Taken when the chunk has enough
 *     queries per row that 2*H*(dqk+dv) flop per (query, row) pair plus 2*H*Lkv*(dn+dv) per row
 *     is less than the absorbed 2*H*(2*Lkv+dr) per pair (about T > 170 at the V3 shape).
 *   q        [T, H, dqk] act: per head [q_nope | RoPE(q_pe)] at the tokens' positions
 *            (mla_qkv_prefill with the tables of positions prefix_len ..).
 *   kv_cache [n_blocks, 1, bs, R] act (read only); rows prefix_len .. prefix_len + T - 1 must
 *            already hold the chunk's own rows (mla_qkv_prefill with slot_mapping).
 *   block_table  int32 [max_blocks]: the sequence's blocks; prefix_len + T <= max_blocks * bs.
 *   o        [T, H, dv] act out.
 * T >= 1, prefix_len >= 0.  Workspace: mla_workspace_size(cfg, MLA_FN_PREFILL_ATTN_PAGED, T,
 * max_blocks * bs), which covers the expanded form's keys and values (about 83 KB per row at
 * the V3 shape) whenever some prefix_len would take it. */
mla_status mla_prefill_attn_paged(const mla_config* cfg, const mla_weights* w, const void* q, int32_t T,
                                  const void* kv_cache, int64_t n_blocks, const int32_t* block_table,
                                  int32_t max_blocks, int32_t prefix_len, void* o, void* ws, size_t ws_bytes,
                                  void* stream);

/* Output projection y = o @ wo ([NeMo-MLA] o_proj; [MlaWeights] wo).
 *   o [M, H*dv] act; y [M, D] act out.  M >= 1. */
mla_status mla_out_proj(const mla_config* cfg, const mla_weights* w, const void* o, int32_t M,
                        void* y, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes entry point `fn` (MLA_FN_*) needs for n rows (T or B or M) and,
 * for MLA_FN_DECODE_ATTN and MLA_FN_PREFILL_ATTN_PAGED, contexts up to max_context tokens.  Returns 0 for an
 * invalid config or fn.  The value depends only on the arguments. */
size_t mla_workspace_size(const mla_config* cfg, int32_t fn, int32_t n, int32_t max_context);

/* Static, human-readable text of a status code. */
const char* mla_status_string(mla_status s);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
