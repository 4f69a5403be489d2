"""Per-entry-point GPU parity against the float64 oracle.

Each entry point gets seeded synthetic inputs of the workload's shape and value
distribution; the oracle sees the same inputs decoded exactly to float64.  Small
cases are compared element by element; full-size cases compare sampled rows
(all heads) the oracle can afford, plus every cache row for the scatter."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from synth import torch_io
from helpers import assert_close, device_weights, lib_config, need_gpu, sentinel_cache

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
# small shapes with the V2/V3 per-head dims (kv_lora 512, nope 128, rope 64, v 128) and ragged sizes
SMALL_V3 = synth.custom(W[4], 101, "small-v3-prefill", hidden=1024, n_heads=16, q_lora_rank=256, T=300)
SMALL_V2 = synth.custom(W[2], 102, "small-v2-prefill", hidden=512, n_heads=16, T=177)
# 10 heads: the prefill attention deals its items over the whole (query tile, head) list
ODD_HEADS = synth.custom(W[4], 109, "odd-heads-prefill", hidden=1024, n_heads=10, q_lora_rank=256, T=4000)
EDGE_DEC16 = synth.custom(W[3], 103, "edge-decode-h16", hidden=1024, n_heads=16, q_lora_rank=256, B=6)
EDGE_DEC128 = synth.custom(W[3], 104, "edge-decode-h128", B=6)
# the same sequences in 32- and 96-token cache blocks (a 32-token attention sub-tile always lies in
# one block; 96 is not a power of two); same number, so the same weights and rows
EDGE_BS32 = synth.custom(W[3], 104, "edge-decode-h128-bs32", B=6, block_size=32)
EDGE_BS96 = synth.custom(W[3], 104, "edge-decode-h128-bs96", B=6, block_size=96)
EDGE_FP8 = synth.custom(W[5], 105, "edge-decode-fp8", B=6)
# fp8 weights at 64 < M <= 1024 (the mid-M fp8 kernel): ragged rows, a partial last column tile of
# the kv segment, the query up-projection unsplit (RoPE fused in the kernel)
MID_FP8 = synth.custom(W[5], 110, "mid-fp8-h16", hidden=1024, n_heads=16, q_lora_rank=256, B=130)
# bf16 projections at 512 < M <= 1024 (the large-tile kernel with few tiles, K split by rounds)
MID_V3 = synth.custom(W[4], 111, "mid-v3-prefill", hidden=1024, n_heads=16, q_lora_rank=256, T=700)
EDGE_CTX = np.array([1, 63, 64, 65, 200, 1000], np.int32)

_cache = {}


def _weights(w):
    if w.number not in _cache:
        _cache.clear()
        host = synth.make_weights(w)
        _cache[w.number] = (host, O.decode_weights(host), device_weights(host))
    return _cache[w.number]


def _sample_rows(T, n_rand=12, seed=0):
    base = {0, 1, 2, 63, 64, 65, 127, 128, T // 2, T - 2, T - 1}
    r = np.random.default_rng(seed)
    base |= set(r.integers(0, T, n_rand).tolist())
    return np.array(sorted(t for t in base if 0 <= t < T))


# ----------------------------------------------------------------------------- qkv prefill
@pytest.mark.parametrize("w", [SMALL_V3, SMALL_V2, MID_V3, W[2], W[4]], ids=lambda w: w.name)
def test_qkv_prefill(w):
    need_gpu()
    import head_latent_attention_amd as mla
    s, T = w.shape, w.T
    print(f"[qkv_prefill] {w.name} T={T}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    xh = synth.make_x(w, T)
    n_blocks = -(-T // s.block_size) + 3
    perm = synth.shuffled_blocks(w.number, "blocks", n_blocks)
    slots = synth.slots_for(perm, np.arange(T), s.block_size)
    if T < 1000:
        slots[5] = -1  # a skipped token
    cache = sentinel_cache(s, n_blocks)
    sentinel = torch_io.bits(cache).reshape(-1)[0]
    cos, sin = mla.rope_cos_sin(np.arange(T), s.qk_rope)
    q = torch_io.empty_act(s.act, (T, s.n_heads, s.qk_head))
    k = torch_io.empty_act(s.act, (T, s.n_heads, s.qk_head))
    v = torch_io.empty_act(s.act, (T, s.n_heads, s.v_dim))
    mla.mla_qkv_prefill(cfg, dw, torch_io.to_device(xh), cos, sin, q, k, v, cache, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    dims = O.dims_of(s)
    x64 = O.decode_tensor(s.act, xh.data)
    rows = _sample_rows(T) if T > 1000 else np.arange(T)
    qr, rr = O.project(Wd, x64[rows], rows, dims)
    Kr, Vr = O.expand_kv(Wd, rr, dims)
    assert_close(torch_io.to_f64(q)[rows], qr, s.act, "q", rows)
    assert_close(torch_io.to_f64(k)[rows], Kr, s.act, "k", rows)
    assert_close(torch_io.to_f64(v)[rows], Vr, s.act, "v", rows)
    # every cache row: the right row in the right slot, nothing else written
    all_rows = O.project_rows(Wd, x64, np.arange(T), dims)
    flat = torch_io.to_f64(cache).reshape(-1, s.row)
    keep = slots >= 0
    assert_close(flat[slots[keep]], all_rows[keep], s.act, "cache rows", np.arange(T)[keep])
    b = torch_io.bits(cache).reshape(-1, s.row)
    untouched = np.setdiff1d(np.arange(b.shape[0]), slots[keep])
    assert (b[untouched] == sentinel).all()


# ----------------------------------------------------------------------------- causal attention
# T=1000 at 128 heads: 128-query tiles, 1024 items over one workgroup per CU (several rounds);
# T=4764: 19 query tiles of 256, so the last round is reversed and half full.  10 heads: the
# list is not split by XCD (one round at T=700; at T=4000, 320 items, the second round partial).
# q_std 8 makes the softmax peaky (score std about 8 in natural-log units): the running maximum
# moves by more than the kernels' lazy-rescale threshold many times along a row.
PREFILL_ATTN_CASES = [(SMALL_V3, 1, 1.0), (SMALL_V3, 17, 1.0), (SMALL_V3, 300, 1.0), (SMALL_V2, 129, 1.0),
                      (W[4], 1000, 1.0), (W[2], 4096, 1.0), (W[4], 4764, 1.0), (W[4], 8192, 1.0), (ODD_HEADS, 700, 1.0),
                      (ODD_HEADS, 4000, 1.0), (SMALL_V3, 300, 8.0), (W[2], 4096, 8.0), (W[4], 8192, 8.0)]


@pytest.mark.parametrize("w,T,q_std", PREFILL_ATTN_CASES,
                         ids=lambda c: (c.name if not isinstance(c, (int, float)) else
                                        (str(c) if isinstance(c, int) else f"qstd{c:g}")))
def test_prefill_attn(w, T, q_std):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[prefill_attn] {w.name} T={T} q_std={q_std}", flush=True)
    cfg = lib_config(s)
    qh = synth.make_normal(w, f"attn.q.{T}", (T, s.n_heads, s.qk_head), std=q_std)
    kh = synth.make_normal(w, f"attn.k.{T}", (T, s.n_heads, s.qk_head))
    vh = synth.make_normal(w, f"attn.v.{T}", (T, s.n_heads, s.v_dim))
    o = torch_io.empty_act(s.act, (T, s.n_heads, s.v_dim))
    mla.mla_prefill_attn(cfg, torch_io.to_device(qh), torch_io.to_device(kh), torch_io.to_device(vh), o)
    torch.cuda.synchronize()
    rows = _sample_rows(T) if T > 1000 else np.arange(T)
    q64, k64, v64 = (O.decode_tensor(s.act, t.data) for t in (qh, kh, vh))
    ref = O.attention(q64[rows], k64, v64, O.softmax_scale(s.qk_nope, s.qk_rope), rows)
    assert_close(torch_io.to_f64(o)[rows], ref, s.act, "o", rows)


# ----------------------------------------------------------------------------- decode front end
@pytest.mark.parametrize("w", [EDGE_DEC16, EDGE_DEC128, EDGE_BS32, EDGE_BS96, W[3], W[5], MID_FP8], ids=lambda w: w.name)
def test_decode_qkv_and_scatter(w):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[decode_qkv] {w.name} B={w.B}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    ctx = EDGE_CTX if w.B == 6 else synth.context_lengths(w)
    pg = synth.make_paging(w.number, ctx, s.block_size)
    slots = synth.decode_slot_mapping(pg)
    cache = sentinel_cache(s, pg.n_blocks)
    sentinel = torch_io.bits(cache[:1]).reshape(-1)[0]
    xh = synth.make_x(w, w.B, "x.decode")
    pos = ctx.astype(np.int64) - 1
    cos, sin = mla.rope_cos_sin(pos, s.qk_rope)
    q = torch_io.empty_act(s.act, (w.B, s.n_heads, s.qk_head))
    mla.mla_decode_qkv_and_scatter(cfg, dw, torch_io.to_device(xh), cos, sin, cache,
                                   torch.from_numpy(slots).cuda(), q)
    torch.cuda.synchronize()
    qr, rr = O.project(Wd, O.decode_tensor(s.act, xh.data), pos, O.dims_of(s))
    assert_close(torch_io.to_f64(q), qr, s.act, "q")
    flat = cache.view(-1, s.row)
    got_rows = torch_io.to_f64(flat[torch.from_numpy(slots.astype(np.int64)).cuda()])
    assert_close(got_rows, rr, s.act, "cache rows")
    # nothing but the B slots was written
    mask = torch.ones(flat.shape[0], dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(slots.astype(np.int64)).cuda()] = False
    rest = flat[mask]
    assert bool((rest.view(torch.int16 if s.act == "bf16" else torch.int32) == int(sentinel)).all())


# ----------------------------------------------------------------------------- absorbed decode attention
def _paged_cache(w, ctx):
    s = w.shape
    pg = synth.make_paging(w.number, ctx, s.block_size)
    host = np.zeros((pg.n_blocks, s.block_size, s.row), np.uint16 if s.act == "bf16" else np.float32)
    for b, n in enumerate(ctx):
        synth.fill_cache(host, pg, b, synth.history_rows(w, b, int(n)).data)
    kind = synth.BF16 if s.act == "bf16" else synth.F32
    dev = torch_io.to_device(synth.Tensor(kind, host)).view(pg.n_blocks, 1, s.block_size, s.row)
    return pg, dev


def _decode_sample(ctx):
    """Sequences the oracle recomputes at full batch: the two shortest, the median, the longest
    (split over the most attention shares) and two seeded random ones."""
    order = np.argsort(ctx, kind="stable")
    pick = {int(order[0]), int(order[1]), int(order[len(order) // 2]), int(np.argmax(ctx))}
    pick |= set(np.random.default_rng(7).choice(len(ctx), 2, replace=False).tolist())
    return np.array(sorted(pick))


# q_std 6.4 (8x the usual 0.8) makes the softmax peaky: the lazy rescale runs along every long
# sequence.
DECODE_ATTN_CASES = [(EDGE_DEC16, 0.8), (EDGE_DEC128, 0.8), (EDGE_BS32, 0.8), (EDGE_BS96, 0.8), (EDGE_FP8, 0.8),
                     (W[3], 0.8), (W[5], 0.8), (EDGE_DEC128, 6.4), (W[3], 6.4)]


@pytest.mark.parametrize("w,q_std", DECODE_ATTN_CASES,
                         ids=lambda c: c.name if not isinstance(c, float) else f"qstd{c:g}")
def test_decode_attn_absorbed(w, q_std):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[decode_attn] {w.name} B={w.B} q_std={q_std}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    ctx = EDGE_CTX if w.B == 6 else synth.context_lengths(w)
    pg, cache = _paged_cache(w, ctx)
    qh = synth.make_normal(w, "decode.q", (w.B, s.n_heads, s.qk_head), std=q_std)
    o = torch_io.empty_act(s.act, (w.B, s.n_heads, s.v_dim))
    mla.mla_decode_attn_absorbed(cfg, dw, torch_io.to_device(qh), cache, torch.from_numpy(pg.block_table).cuda(),
                                 torch.from_numpy(ctx).cuda(), o)
    torch.cuda.synchronize()
    bs_ = np.arange(w.B) if w.B <= 8 else _decode_sample(ctx)
    q64 = O.decode_tensor(s.act, qh.data)
    seqs = [O.decode_tensor(s.act, synth.history_rows(w, int(b), int(ctx[b])).data) for b in bs_]
    ref = O.decode_attention(Wd, q64[bs_], seqs, O.dims_of(s))
    assert_close(torch_io.to_f64(o)[bs_], ref, s.act, f"o (sequences {bs_.tolist()}, contexts {ctx[bs_].tolist()})",
                 bs_)


# Few long sequences: each one split across many attention shares, so the combine merges up to
# 256 partial results per head and sequence (B = 1, 16384 tokens: exactly one 64-token tile per
# share; B = 2: about 128 shares per sequence).  The weights are those of the full-size decode
# workload (same shapes; the cases above leave them cached).
LONG_ONE = synth.custom(W[3], 112, "long-one-h128", B=1, ctx_lo=16384, ctx_hi=16384)
LONG_TWO = synth.custom(W[3], 113, "long-two-h128", B=2, ctx_lo=9000, ctx_hi=13000)


@pytest.mark.parametrize("w", [LONG_ONE, LONG_TWO], ids=lambda w: w.name)
def test_decode_attn_long_split(w):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    host, Wd, dw = _weights(W[3])
    cfg = lib_config(s)
    ctx = synth.context_lengths(w)
    print(f"[decode_attn_long] {w.name} B={w.B} contexts {ctx.tolist()}", flush=True)
    pg, cache = _paged_cache(w, ctx)
    qh = synth.make_normal(w, "decode.q", (w.B, s.n_heads, s.qk_head), std=0.8)
    o = torch_io.empty_act(s.act, (w.B, s.n_heads, s.v_dim))
    mla.mla_decode_attn_absorbed(cfg, dw, torch_io.to_device(qh), cache, torch.from_numpy(pg.block_table).cuda(),
                                 torch.from_numpy(ctx).cuda(), o)
    torch.cuda.synchronize()
    bs_ = np.arange(w.B)
    q64 = O.decode_tensor(s.act, qh.data)
    seqs = [O.decode_tensor(s.act, synth.history_rows(w, int(b), int(ctx[b])).data) for b in bs_]
    ref = O.decode_attention(Wd, q64, seqs, O.dims_of(s))
    assert_close(torch_io.to_f64(o), ref, s.act, f"o (contexts {ctx.tolist()})", bs_)


# Many short sequences: several whole sequences inside one attention workgroup's share of the
# 64-token tile list (so partial results are written and queries reloaded several times per
# workgroup), and more sequences than the planner keeps in LDS (its global-memory path).
SHORT_MANY = synth.custom(W[3], 107, "short-many-h128", B=700, ctx_lo=1, ctx_hi=150)
SHORT_HUGE_B = synth.custom(W[3], 108, "short-b2100-h128", B=2100, ctx_lo=1, ctx_hi=40)
ATTN_SHARES = 256  # workgroups of the decode attention: the tile list is cut into this many shares


def _share_sample(ctx, n_pick=10):
    """Sequences at interesting places of the share split: the first and last, ones a share
    boundary cuts, and ones that share a workgroup with other whole sequences."""
    tiles = -(-ctx.astype(np.int64) // 64)
    P = np.concatenate([[0], np.cumsum(tiles)])
    N = int(P[-1])
    bounds = [(r * N) // ATTN_SHARES for r in range(ATTN_SHARES + 1)]
    cut = [b for b in range(len(ctx)) if any(P[b] < x < P[b + 1] for x in bounds)]
    share_of = np.searchsorted(bounds, P[:-1], side="right") - 1
    crowded = [b for b in range(len(ctx)) if np.count_nonzero(share_of == share_of[b]) >= 3]
    pick = {0, len(ctx) - 1} | set(cut[:n_pick // 2]) | set(crowded[:: max(1, len(crowded) // (n_pick // 2))][:n_pick // 2])
    return np.array(sorted(pick))


@pytest.mark.parametrize("w", [SHORT_MANY, SHORT_HUGE_B], ids=lambda w: w.name)
def test_decode_attn_many_short_sequences(w):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[decode_attn_short] {w.name} B={w.B}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    ctx = synth.context_lengths(w)
    pg, cache = _paged_cache(w, ctx)
    qh = synth.make_normal(w, "decode.q", (w.B, s.n_heads, s.qk_head), std=0.8)
    o = torch_io.empty_act(s.act, (w.B, s.n_heads, s.v_dim))
    mla.mla_decode_attn_absorbed(cfg, dw, torch_io.to_device(qh), cache, torch.from_numpy(pg.block_table).cuda(),
                                 torch.from_numpy(ctx).cuda(), o)
    torch.cuda.synchronize()
    bs_ = _share_sample(ctx)
    q64 = O.decode_tensor(s.act, qh.data)
    seqs = [O.decode_tensor(s.act, synth.history_rows(w, int(b), int(ctx[b])).data) for b in bs_]
    ref = O.decode_attention(Wd, q64[bs_], seqs, O.dims_of(s))
    assert_close(torch_io.to_f64(o)[bs_], ref, s.act, f"o (sequences {bs_.tolist()})", bs_)
    # every output is finite (a share's partial written to a wrong slot would leave garbage)
    assert torch.isfinite(o.float()).all()


# ----------------------------------------------------------------------------- output projection
@pytest.mark.parametrize("w,M", [(SMALL_V3, 300), (EDGE_FP8, 7), (W[2], 4096), (W[3], 64), (W[4], 8192), (W[5], 256),
                                 (MID_FP8, 300), (W[5], 1000), (MID_V3, 700), (W[4], 1000), (W[4], 8000)],
                         ids=lambda c: str(c) if isinstance(c, int) else c.name)
def test_out_proj(w, M):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[out_proj] {w.name} M={M}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    oh = synth.make_normal(w, f"oproj.o.{M}", (M, s.n_heads * s.v_dim), std=0.5)
    y = torch_io.empty_act(s.act, (M, s.hidden))
    mla.mla_out_proj(cfg, dw, torch_io.to_device(oh), y)
    torch.cuda.synchronize()
    rows = _sample_rows(M) if M > 1000 else np.arange(M)
    if M > 1000:
        # both sides of every 256-row tile edge in the bottom row tiles of the large-tile GEMM
        # (the last one ragged at M = 8000)
        last = (M - 1) // 256
        edges = [e for t in range(max(1, last - 6), last + 1) for e in (256 * t - 1, 256 * t)]
        rows = np.union1d(rows, [e for e in edges if e < M])
    ref = O.decode_tensor(s.act, oh.data)[rows] @ Wd["wo"]
    assert_close(torch_io.to_f64(y)[rows], ref, s.act, "y", rows)
