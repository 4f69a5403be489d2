"""Plain float64 CPU oracle of DeepSeek-V2/V3 multi-head latent attention (MLA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``.  It shares no code with the HIP library and never reads
anything the HIP library produced.

The oracle computes the layer the *expanded* way: every head's key and value
are materialised from the latent rows through ``wkv_b`` and ordinary softmax
attention runs per head.  No absorption, blocking or fusion is applied.  All
arithmetic is numpy float64; matrix products use numpy's ``@``.

Page references (titles of the source pages):
  [NeMo-MLA]   NVIDIA NeMo AutoModel, nemo_automodel.components.models.deepseek_v3.layers, class MLA
  [Mla]        logicaffeine_compile, model::spec, Struct Mla
  [MlaWeights] atlas docs, spark_model::layers::qwen3_attention, Struct MlaWeights
  [NKI-Decode] AWS Neuron NKI, "MLA Decode QKV Kernel API Reference"
  [NKI-CTE]    AWS Neuron NKI, "QKV CTE MLA Kernel API Reference"
  [YaRN]       Peng, Quesnelle, Fan, Shippole, "YaRN: Efficient Context Window Extension
               of Large Language Models" (2023), the published method the [Mla] scale
               and the [MlaWeights] yarn_inv_freq table refer to

Readings where the pages are silent (each listed in the design notes too):
  * RMSNorm is x * (mean(x^2) + eps)^-1/2 * gamma with gamma used as is.
  * RoPE rotates element pair (2i, 2i+1) as the complex number x_2i + j x_2i+1
    multiplied by exp(j * pos * theta^(-2i/qk_rope)), theta = 10000.
  * The cached row is [normalised c_kv | roped k_pe]; k_pe is not normalised.
  * Positions are 0-based; a decode token at position ctx-1 attends to all ctx
    rows including its own.
  * YaRN: pair i keeps its frequency while its wavelength fits at least beta_fast
    times into the original context, is divided by the extension factor once it
    fits at most beta_slow times, and in between is blended with a weight that is
    linear in the pair index (the pair bounds rounded outward); the magnitude
    0.1*m*ln(factor)+1 enters the score scale squared and leaves cos/sin unscaled.
  * The optional layer-input RMSNorm (input_norm_w) uses the same formula and eps
    as the two latent norms and is applied to x before the stage-1 projection.
  * fp8 activation quantisation (when dims["act_quant"] is set): every activation
    entering a projection (x, the normed q latent, the normed kv latent, the
    attention output), as the bf16 value the layer stores, is quantised per token and
    per group of 128 columns to E4M3FN codes times a power-of-two scale 2^e, e the
    smallest integer with max|group| <= 448 * 2^e, codes rounded to nearest, ties to even.

Parity pins: every function here is checked in tests/test_oracle_*.py against
closed forms, textbook special cases, torch's CPU float8 decoding, or
pure-Python brute force on tiny shapes.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "e4m3fn_value", "e4m3fn_round", "bf16_round", "quantize_mx_fp8", "decode_tensor", "rms_norm", "rope_angles", "rope_interleaved",
    "softmax_scale", "yarn_inv_freq", "yarn_mscale", "input_norm", "project", "project_rows", "expand_kv", "attention", "mla_prefill", "mla_decode", "decode_attention", "chunk_attention",
    "out_proj", "place_rows", "cache_read_dense", "decode_weights", "dims_of",
]


# ----------------------------------------------------------------------------- storage formats
def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN code: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Subnormals (exponent field 0) are m * 2^-9; S.1111.111 is NaN; there is no
    infinity, so the largest finite magnitude is S.1111.110 = 448.
    [MlaWeights] fp8 fields: weights ship as FP8-E4M3 with 128x128 block scales."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_round(v: np.ndarray) -> np.ndarray:
    """E4M3FN code of the representable value nearest to each v (|v| <= 448), ties to the
    code with an even mantissa (round to nearest even); the sign of zero is kept."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > 448.0) or np.any(np.isnan(v)):
        raise ValueError("value outside the E4M3FN range")
    mags = np.array([e4m3fn_value(c) for c in range(0x7F)])          # codes 0x00..0x7E, increasing
    a = np.abs(v).reshape(-1)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)     # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == mags[hi], hi, np.where(pick_hi, hi, lo))
    sign = np.signbit(v.reshape(-1)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8).reshape(v.shape)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (8-bit mantissa), ties to even, of each float64 v (finite)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)   # np.round rounds halves to even


def quantize_mx_fp8(x: np.ndarray, group: int = 128):
    """Per-row, per-group fp8 quantisation with power-of-two scales.

    [NKI-CTE] quantises activations to MX fp8 with 8-bit power-of-two (compact) scales;
    the group is 128 columns of one token (the weights' 128 block size along K).  For
    each group the exponent e is the smallest integer with max|x| <= 448 * 2^e (0 for an
    all-zero group, clamped to [-127, 127]) and codes = E4M3FN(x * 2^-e).  Returns (codes uint8 [M, K],
    exponents int [M, ceil(K/group)], dequantised float64 [M, K])."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    G = -(-K // group)
    exps = np.zeros((M, G), dtype=np.int64)
    codes = np.zeros((M, K), dtype=np.uint8)
    for gi in range(G):
        blk = x[:, gi * group:(gi + 1) * group]
        for m in range(M):
            amax = float(np.max(np.abs(blk[m])))
            if amax == 0.0:
                continue
            mant, ex = math.frexp(amax)           # amax = mant * 2^ex, mant in [0.5, 1)
            e = ex - 9                            # 448 = 0.875 * 2^9
            if amax > 448.0 * 2.0 ** e:
                e += 1
            exps[m, gi] = min(max(e, -127), 127)   # the range of an 8-bit power-of-two (E8M0) scale
        codes[:, gi * group:(gi + 1) * group] = e4m3fn_round(blk * 2.0 ** (-exps[:, gi:gi + 1]))
    table = np.array([e4m3fn_value(c) for c in range(256)])
    deq = table[codes] * 2.0 ** np.repeat(exps, group, axis=1)[:, :K]
    return codes, exps, deq


def _act(a: np.ndarray, dims: dict) -> np.ndarray:
    """An activation as a projection consumes it: fp8-quantised and dequantised when the
    layer quantises activations (dims["act_quant"]), else unchanged.  The quantiser sees a
    bfloat16 tensor: the MX projection of "QKV CTE MLA Kernel API Reference" (qkv_mla_mx,
    Parameters and Returns) keeps x, the normed Q and KV intermediates (their RMSNorm gammas
    are bf16) and every output in bf16, so each input it quantises is a bf16 value.  Each
    code is a decision taken in floating point, made here on that same bf16 value."""
    if not dims.get("act_quant"):
        return a
    shape = a.shape
    return quantize_mx_fp8(bf16_round(a.reshape(-1, shape[-1])))[2].reshape(shape)


def decode_tensor(kind: str, data: np.ndarray, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Exact float64 value of a host array in the library's storage format.

    f32: the float32 values; bf16: uint16 patterns are the top half of a float32;
    fp8: E4M3FN code value times its block's fp32 scale, the block being 128x128
    over a [K, N] weight ([NKI-CTE] scale shapes [K/128, ceil(N/128)];
    [MlaWeights] fp8 fields: the dequantisation multiplies by the block scale)."""
    if kind == "f32":
        return np.asarray(data, dtype=np.float32).astype(np.float64)
    if kind == "bf16":
        u = np.asarray(data, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    if kind == "fp8":
        vals = _E4M3FN_TABLE[np.asarray(data, dtype=np.uint8)]
        K, N = vals.shape
        s = np.asarray(scale, dtype=np.float64)
        rows = np.arange(K) // 128
        cols = np.arange(N) // 128
        return vals * s[rows][:, cols]
    raise ValueError(kind)


# ----------------------------------------------------------------------------- elementary steps
def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, times gamma.

    [NKI-Decode] Parameters: q_norm_w / kv_norm_w are the RMSNorm gammas of the
    query latent and the KV latent, norm_eps defaults to 1e-6.
    [Mla] description: the shared latent is RMS-normed."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def rope_angles(positions: np.ndarray, rope_dim: int, theta: float = 10000.0,
                inv_freq: Optional[np.ndarray] = None) -> np.ndarray:
    """Angle of pair i at each position: pos * inv_freq[i], shape [T, rope_dim/2].

    Without a table inv_freq[i] = theta^(-2i/rope_dim) ([MlaWeights] main_inv_freq:
    the plain theta = 10000 inverse frequencies with no YaRN); a given table is
    used as is ([MlaWeights] yarn_inv_freq)."""
    if inv_freq is None:
        i = np.arange(rope_dim // 2, dtype=np.float64)
        inv_freq = theta ** (-2.0 * i / rope_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * np.asarray(inv_freq, np.float64)[None, :]


def yarn_inv_freq(rope_dim: int, theta: float, factor: float, original_max_position: int,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """YaRN inverse frequencies [rope_dim/2] ([YaRN] section 3.2, interpolation by parts).

    A pair whose wavelength 2*pi/f_i fits at least beta_fast times into the original
    context keeps f_i; one that fits at most beta_slow times is interpolated to
    f_i/factor; in between the two are blended.  The pair index at which the count
    equals n solves original_max_position * f_i / (2*pi) = n; the blend weight is
    linear in the pair index between floor(index(beta_fast)) (clamped at 0) and
    ceil(index(beta_slow)) (clamped at rope_dim-1).  factor <= 1 is plain RoPE."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    plain = theta ** (-2.0 * i / rope_dim)
    if factor <= 1.0:
        return plain

    def pair_index(rotations: float) -> float:
        return rope_dim * math.log(original_max_position / (rotations * 2.0 * math.pi)) / (2.0 * math.log(theta))

    lo = max(math.floor(pair_index(beta_fast)), 0)
    hi = min(math.ceil(pair_index(beta_slow)), rope_dim - 1)
    if hi > lo:
        w_interp = np.clip((i - lo) / (hi - lo), 0.0, 1.0)
    else:
        w_interp = (i > lo).astype(np.float64)
    return plain / factor * w_interp + plain * (1.0 - w_interp)


def yarn_mscale(factor: float, m: float = 1.0) -> float:
    """YaRN's attention magnitude 0.1 * m * ln(factor) + 1 ([YaRN] section 3.4), 1 for factor <= 1."""
    return 1.0 if factor <= 1.0 else 0.1 * m * math.log(factor) + 1.0


def rope_interleaved(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Interleaved rotary embedding over the last axis.

    x: [T, ..., rope_dim]; angles: [T, rope_dim/2].  Element 2i pairs with
    element 2i+1 ([NKI-Decode] Notes: interleaved RoPE, not the half-split
    pairing of the sparse indexer), rotated as a complex number by the angle
    ([NeMo-MLA] forward takes complex freqs_cis)."""
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    z = x.reshape(shape[:-1] + (shape[-1] // 2, 2))
    a = angles.reshape((angles.shape[0],) + (1,) * (x.ndim - 2) + (angles.shape[1],))
    c, s = np.cos(a), np.sin(a)
    re = z[..., 0] * c - z[..., 1] * s
    im = z[..., 0] * s + z[..., 1] * c
    return np.stack([re, im], axis=-1).reshape(shape)


def softmax_scale(qk_nope: int, qk_rope: int, rope_factor: float = 1.0, mscale_all_dim: float = 1.0) -> float:
    """[NeMo-MLA] softmax_scale = qk_head_dim ** -0.5; [Mla] scale: 1/sqrt(qk_nope + qk_rope)
    times the square of YaRN's magnitude (which is 1 without YaRN)."""
    return yarn_mscale(rope_factor, mscale_all_dim) ** 2 / math.sqrt(qk_nope + qk_rope)


def input_norm(W: Dict[str, np.ndarray], x: np.ndarray, dims: dict) -> np.ndarray:
    """The layer's input RMSNorm when an input_norm_w gamma [hidden] is given, else x
    ([NKI-Decode] input_norm_w: folded into the hidden load; norm_eps is the epsilon of
    every RMSNorm of that kernel)."""
    if "input_norm_w" not in W:
        return x
    return rms_norm(x, W["input_norm_w"], dims["norm_eps"])


# ----------------------------------------------------------------------------- projections
def project(W: Dict[str, np.ndarray], x: np.ndarray, positions: np.ndarray, dims: dict):
    """Query and cache-row front end for tokens x [T, hidden] at the given positions.

    Stage 1 ([NKI-CTE] Notes, combined Q/KV path stage 1 and its split):
        x @ wq_a -> q latent,  x @ wkv_a -> [c_kv | k_pe].
    Q path stage 2: RMSNorm(q latent) @ wq_b; with no q latent ([Mla] q_lora_rank
    is optional) the query is x @ wq_b directly.
    Per head the query is [q_nope | q_pe] ([NKI-Decode] wq_b parameter).
    RoPE on each head's trailing qk_rope dims and once on k_pe ([Mla] description:
    the rope key is shared by every head; [NKI-CTE] final assembly).

    With input_norm_w in W, x first goes through the layer's input RMSNorm.

    Returns q [T, H, dqk] (q_pe roped) and rows [T, kv_lora + qk_rope] = [c_norm | k_pe roped].
    """
    H, dn, dr, Lkv = dims["n_heads"], dims["qk_nope"], dims["qk_rope"], dims["kv_lora_rank"]
    eps = dims["norm_eps"]
    ang = rope_angles(positions, dr, dims.get("rope_theta", 10000.0), dims.get("inv_freq"))
    rows = project_rows(W, x, positions, dims)
    x = _act(input_norm(W, x, dims), dims)
    if "wq_a" in W:
        cq = rms_norm(x @ W["wq_a"], W["q_norm_w"], eps)
        q = _act(cq, dims) @ W["wq_b"]
    else:
        q = x @ W["wq_b"]
    q = q.reshape(x.shape[0], H, dn + dr)
    q = np.concatenate([q[..., :dn], rope_interleaved(q[..., dn:], ang)], axis=-1)
    return q, rows


def project_rows(W: Dict[str, np.ndarray], x: np.ndarray, positions: np.ndarray, dims: dict) -> np.ndarray:
    """Latent-cache rows of tokens x [T, hidden]: [RMSNorm(c_kv) | RoPE(k_pe)].

    x @ wkv_a gives one cache row per token split as [c_kv | k_pe] ([NKI-Decode]
    wkv_a parameter; [NKI-CTE] stage-1 split); the latent is RMS-normed with
    kv_norm_w, the rope key rotated at the token's position and not normed.  x is
    first put through the layer-input RMSNorm when W holds input_norm_w."""
    Lkv, dr = dims["kv_lora_rank"], dims["qk_rope"]
    ang = rope_angles(positions, dr, dims.get("rope_theta", 10000.0), dims.get("inv_freq"))
    kva = _act(input_norm(W, x, dims), dims) @ W["wkv_a"]
    c = rms_norm(kva[:, :Lkv], W["kv_norm_w"], dims["norm_eps"])
    p = rope_interleaved(kva[:, Lkv:], ang)
    return np.concatenate([c, p], axis=-1)


def expand_kv(W: Dict[str, np.ndarray], rows: np.ndarray, dims: dict):
    """Per-head keys and values from latent rows [T, R].

    [NKI-CTE] KV path stage 2: norm(c_kv) @ wkv_b split per head into
    [k_nope | v]; final assembly: K = [k_nope | k_pe broadcast to every head].
    Returns K [T, H, dqk], V [T, H, dv]."""
    H, dn, dv, Lkv = dims["n_heads"], dims["qk_nope"], dims["v_dim"], dims["kv_lora_rank"]
    T = rows.shape[0]
    kv = (_act(rows[:, :Lkv], dims) @ W["wkv_b"]).reshape(T, H, dn + dv)
    p = np.broadcast_to(rows[:, None, Lkv:], (T, H, rows.shape[1] - Lkv))
    return np.concatenate([kv[..., :dn], p], axis=-1), kv[..., dn:].copy()


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              q_positions: np.ndarray) -> np.ndarray:
    """softmax(scale * q K^T) V per head, query i seeing key positions j <= q_positions[i].

    q [Tq, H, dqk], K [Tk, H, dqk], V [Tk, H, dv] -> [Tq, H, dv].  The softmax
    subtracts the row maximum before exponentiating ([NeMo-MLA] forward with a
    causal attention_mask; softmax_scale attribute)."""
    s = np.matmul(q.transpose(1, 0, 2), K.transpose(1, 2, 0)) * scale     # [H, Tq, Tk]
    j = np.arange(K.shape[0])
    mask = j[None, :] > np.asarray(q_positions)[:, None]
    s = np.where(mask[None], -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.matmul(p, V.transpose(1, 0, 2)).transpose(1, 0, 2)          # [Tq, H, dv]


def out_proj(W: Dict[str, np.ndarray], o: np.ndarray, dims: dict) -> np.ndarray:
    """y = concat_h(o) @ wo ([NeMo-MLA] o_proj), o quantised first when the layer quantises
    activations."""
    return _act(o.reshape(o.shape[0], -1), dims) @ W["wo"]


# ----------------------------------------------------------------------------- whole layer
def mla_prefill(W: Dict[str, np.ndarray], x: np.ndarray, dims: dict) -> dict:
    """Causal prefill of T tokens at positions 0..T-1 of one sequence.

    Returns q, k, v (the per-head tensors the context-encoding QKV kernel emits,
    [NKI-CTE] return values), rows (cache rows), o [T, H, dv] and
    y = concat_h(o) @ wo [T, hidden] ([NeMo-MLA] o_proj)."""
    T = x.shape[0]
    pos = np.arange(T)
    q, rows = project(W, x, pos, dims)
    K, V = expand_kv(W, rows, dims)
    o = attention(q, K, V, dims["softmax_scale"], pos)
    y = out_proj(W, o, dims)
    return dict(q=q, k=K, v=V, rows=rows, o=o, y=y)


def mla_decode(W: Dict[str, np.ndarray], x: np.ndarray, history: Sequence[np.ndarray],
               dims: dict, head_chunk: int = 16) -> dict:
    """One decode step for B sequences; sequence b has len(history[b]) earlier rows.

    The new token sits at position len(history[b]); its row is appended and it
    attends to every row including its own.  Keys and values are expanded per
    head through wkv_b (head_chunk heads at a time to bound memory).
    Returns q [B, H, dqk], rows [B, R], o [B, H, dv], y [B, hidden]."""
    B = x.shape[0]
    pos = np.array([len(h) for h in history])
    q, rows = project(W, x, pos, dims)
    seqs = [np.concatenate([np.asarray(history[b], dtype=np.float64).reshape(-1, rows.shape[1]),
                            rows[b:b + 1]], axis=0) for b in range(B)]
    o = decode_attention(W, q, seqs, dims, head_chunk)
    y = out_proj(W, o, dims)
    return dict(q=q, rows=rows, o=o, y=y)


def decode_attention(W: Dict[str, np.ndarray], q: np.ndarray, seqs: Sequence[np.ndarray], dims: dict,
                     head_chunk: int = 16) -> np.ndarray:
    """Attention of one query per sequence over all of that sequence's latent rows.

    q [B, H, dqk] (q_pe already roped); seqs[b] = rows [n_b, R] of sequence b
    (the query's own row last).  Keys and values are expanded per head through
    wkv_b ([NKI-CTE] KV path stage 2 and final assembly), head_chunk heads at a
    time; the latent rows are not quantised (absorbed attention has no projection
    input).  Returns o [B, H, dv]."""
    H, dv = dims["n_heads"], dims["v_dim"]
    B = q.shape[0]
    o = np.zeros((B, H, dv))
    for b in range(B):
        rows = np.asarray(seqs[b], dtype=np.float64)
        for h0 in range(0, H, head_chunk):
            hs = slice(h0, min(H, h0 + head_chunk))
            sub = _head_slice(W, dims, hs)
            K, V = expand_kv(sub, rows, dict(dims, n_heads=hs.stop - hs.start, act_quant=False))
            o[b, hs] = attention(q[b:b + 1, hs], K, V, dims["softmax_scale"], np.array([len(rows) - 1]))[0]
    return o


def chunk_attention(W: Dict[str, np.ndarray], q: np.ndarray, prefix_rows: np.ndarray, chunk_rows: np.ndarray,
                    dims: dict, head_chunk: int = 16) -> np.ndarray:
    """Causal attention of a prefill chunk over an existing prefix of one sequence.

    q [T, H, dqk] are the chunk's queries at positions P..P+T-1 (P = len(prefix_rows),
    q_pe roped there); prefix_rows [P, R] and chunk_rows [T, R] are the sequence's latent
    rows.  Query t sees rows 0..P+t.  Keys and values of every row are expanded per head
    through wkv_b ([NKI-CTE] KV path stage 2 and final assembly), as in the whole-prompt
    prefill ([NeMo-MLA] forward, causal mask).  Returns o [T, H, dv]."""
    H, dv = dims["n_heads"], dims["v_dim"]
    rows = np.concatenate([np.asarray(prefix_rows, np.float64).reshape(-1, chunk_rows.shape[1]),
                           np.asarray(chunk_rows, np.float64)], axis=0)
    P, T = rows.shape[0] - chunk_rows.shape[0], q.shape[0]
    o = np.zeros((T, H, dv))
    for h0 in range(0, H, head_chunk):
        hs = slice(h0, min(H, h0 + head_chunk))
        sub = _head_slice(W, dims, hs)
        K, V = expand_kv(sub, rows, dict(dims, n_heads=hs.stop - hs.start, act_quant=False))
        o[:, hs] = attention(q[:, hs], K, V, dims["softmax_scale"], P + np.arange(T))
    return o


def _head_slice(W, dims, hs: slice) -> dict:
    w = dims["qk_nope"] + dims["v_dim"]
    return {"wkv_b": W["wkv_b"][:, hs.start * w:hs.stop * w]}


# ----------------------------------------------------------------------------- paged cache
def place_rows(cache: np.ndarray, slot_mapping: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Expected cache after writing row t to flat slot slot_mapping[t] ([NKI-Decode]
    kv_cache / slot_mapping parameters); slot -1 skips the token."""
    out = cache.copy()
    flat = out.reshape(-1, out.shape[-1])
    for t, s in enumerate(np.asarray(slot_mapping)):
        if s >= 0:
            flat[s] = rows[t]
    return out


def cache_read_dense(cache: np.ndarray, block_table_row: np.ndarray, n: int, block_size: int) -> np.ndarray:
    """Rows 0..n-1 of one sequence read back through its block table (logical row t
    lives in physical block block_table_row[t // block_size] at offset t % block_size)."""
    out = np.empty((n, cache.shape[-1]), dtype=cache.dtype)
    for t in range(n):
        out[t] = cache[block_table_row[t // block_size], t % block_size]
    return out


def decode_weights(tensors: dict) -> Dict[str, np.ndarray]:
    """float64 views of every weight/gamma of a synth weight dict."""
    out = {}
    for name, t in tensors.items():
        out[name] = decode_tensor(t.kind, t.data, t.scale)
    return out


def dims_of(shape) -> dict:
    """The scalar parameters of a layer as a plain dict (names follow [NKI-Decode] /
    [NKI-CTE] parameters).  With a YaRN factor above 1 the dict also holds the
    YaRN inverse-frequency table and the score scale includes YaRN's magnitude."""
    factor = getattr(shape, "rope_factor", 1.0)
    d = dict(hidden=shape.hidden, n_heads=shape.n_heads, q_lora_rank=shape.q_lora_rank,
             kv_lora_rank=shape.kv_lora_rank, qk_nope=shape.qk_nope, qk_rope=shape.qk_rope,
             v_dim=shape.v_dim, norm_eps=shape.norm_eps, rope_theta=shape.rope_theta,
             softmax_scale=softmax_scale(shape.qk_nope, shape.qk_rope, factor,
                                         getattr(shape, "rope_mscale_all_dim", 1.0)),
             act_quant=bool(getattr(shape, "act_quant", False)))
    if factor > 1.0:
        d["inv_freq"] = yarn_inv_freq(shape.qk_rope, shape.rope_theta, factor, shape.rope_original_max,
                                      shape.rope_beta_fast, shape.rope_beta_slow)
    return d
