"""GPU parity of the rotary-table builders and of the projection and attention entry
points with YaRN frequencies, YaRN's score scale and the layer-input RMSNorm.

Tables come from mla_rope_inv_freq / mla_rope_tables on the device; the oracle builds
its own angles in float64 from the YaRN definition.  Positions reach well past the
original context (4096), where the YaRN blend matters."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from synth import torch_io
from helpers import assert_close, device_weights, lib_config, need_gpu, sentinel_cache

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
YARN_V3 = dict(rope_factor=40.0)
ROPES = [  # (qk_rope, theta, factor, original context, beta_fast, beta_slow, m)
    (64, 1e4, 1.0, 4096, 32.0, 1.0, 1.0),
    (64, 1e4, 40.0, 4096, 32.0, 1.0, 1.0),
    (128, 5e5, 8.0, 8192, 16.0, 2.0, 0.707),
    (16, 1e4, 8.0, 256, 32.0, 1.0, 1.0),
]
POSITIONS = np.array([0, 1, 2, 63, 4095, 4096, 4097, 9000, 32767, 100000, 163839, 1 << 20], np.int32)


def _lib_rope(shape):
    import head_latent_attention_amd as mla
    return mla.rope(theta=shape.rope_theta, factor=shape.rope_factor, original_max_position=shape.rope_original_max,
                    beta_fast=shape.rope_beta_fast, beta_slow=shape.rope_beta_slow,
                    mscale_all_dim=shape.rope_mscale_all_dim)


def _cfg(shape):
    import head_latent_attention_amd as mla
    return mla.config(shape.hidden, shape.n_heads, shape.q_lora_rank, shape.kv_lora_rank, shape.qk_nope,
                      shape.qk_rope, shape.v_dim, act=shape.act, weight=shape.weight, block_size=shape.block_size,
                      norm_eps=shape.norm_eps, rope=_lib_rope(shape))


def _tables(shape, positions, pos_offset=0):
    import head_latent_attention_amd as mla
    inv = mla.mla_rope_inv_freq(_lib_rope(shape), shape.qk_rope)
    pos = torch.from_numpy(np.asarray(positions, np.int32)).cuda()
    return mla.mla_rope_tables(pos, pos.numel(), shape.qk_rope, inv, pos_offset=pos_offset)


@pytest.mark.parametrize("r", ROPES, ids=lambda r: f"dr{r[0]}-theta{r[1]:g}-s{r[2]:g}")
def test_rope_inv_freq_and_tables(r):
    need_gpu()
    import head_latent_attention_amd as mla
    dr, theta, s, L, bf, bs, m = r
    print(f"[rope] dr={dr} theta={theta} factor={s}", flush=True)
    inv = mla.mla_rope_inv_freq(mla.rope(theta, s, L, bf, bs, m), dr)
    ref = O.yarn_inv_freq(dr, theta, s, L, bf, bs)
    got = inv.cpu().numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=0), np.max(np.abs(got / ref - 1))
    # tables at decode positions given as context lengths (offset -1)
    ctx = torch.from_numpy(POSITIONS + 1).cuda()
    cos, sin = mla.mla_rope_tables(ctx, len(POSITIONS), dr, inv, pos_offset=-1)
    ang = O.rope_angles(POSITIONS, dr, inv_freq=ref)
    ec = np.max(np.abs(cos.cpu().numpy() - np.cos(ang)))
    es = np.max(np.abs(sin.cpu().numpy() - np.sin(ang)))
    print(f"  cos err {ec:.2e}, sin err {es:.2e}", flush=True)
    # fp32 rounding of values in [-1, 1] plus the angle's fp64 rounding at position 2^20
    assert ec < 2e-7 and es < 2e-7
    if s <= 1.0 and theta == 1e4:  # no table: theta = 10000 frequencies in the kernel
        c2, s2 = mla.mla_rope_tables(None, 9, dr, None)
        a2 = O.rope_angles(np.arange(9), dr)
        assert np.max(np.abs(c2.cpu().numpy() - np.cos(a2))) < 2e-7
        assert np.max(np.abs(s2.cpu().numpy() - np.sin(a2))) < 2e-7


# small V3-per-head shapes with YaRN at the published V3 settings and the layer-input norm
YN_PREFILL = synth.custom(W[4], 130, "yarn-norm-prefill", hidden=1024, n_heads=16, q_lora_rank=256, T=300,
                          input_norm=True, **YARN_V3)
YN_PREFILL_WIDE = synth.custom(W[4], 131, "yarn-norm-prefill-d8448", hidden=8448, n_heads=8, q_lora_rank=256,
                               T=40, input_norm=True, **YARN_V3)
YN_PREFILL_ODD = synth.custom(W[4], 132, "norm-prefill-d1020", hidden=1020, n_heads=4, q_lora_rank=128, T=33,
                              input_norm=True)
YN_TINY = synth.custom(W[1], 133, "yarn-norm-tiny-fp32", input_norm=True, rope_factor=8.0, rope_original_max=256)
YN_DECODE = synth.custom(W[3], 134, "yarn-norm-decode", hidden=1024, n_heads=16, q_lora_rank=256, B=6,
                         input_norm=True, **YARN_V3)
YN_DECODE_V3 = synth.custom(W[3], 135, "yarn-norm-decode-v3", B=6, input_norm=True, **YARN_V3)
YN_CTX = {YN_DECODE.number: np.array([1, 4095, 4097, 9000, 20000, 65], np.int32),
          YN_DECODE_V3.number: np.array([1, 4095, 4097, 5000, 300, 65], np.int32)}


@pytest.mark.parametrize("w", [YN_PREFILL, YN_PREFILL_WIDE, YN_PREFILL_ODD, YN_TINY], ids=lambda w: w.name)
def test_qkv_prefill_yarn_input_norm(w):
    need_gpu()
    import head_latent_attention_amd as mla
    s, T = w.shape, w.T
    print(f"[qkv_prefill+yarn+norm] {w.name} T={T} D={s.hidden}", flush=True)
    host = synth.make_weights(w)
    Wd, dw = O.decode_weights(host), device_weights(host)
    cfg = _cfg(s)
    xh = synth.make_x(w, T)
    n_blocks = -(-T // s.block_size) + 2
    slots = synth.slots_for(synth.shuffled_blocks(w.number, "blocks", n_blocks), np.arange(T), s.block_size)
    cache = sentinel_cache(s, n_blocks)
    # positions 5000.. so the YaRN blend is exercised: tables for positions p0 + t
    p0 = 5000
    cos, sin = _tables(s, np.arange(T) + p0)
    q = torch_io.empty_act(s.act, (T, s.n_heads, s.qk_head))
    k = torch_io.empty_act(s.act, (T, s.n_heads, s.qk_head))
    v = torch_io.empty_act(s.act, (T, s.n_heads, s.v_dim))
    mla.mla_qkv_prefill(cfg, dw, torch_io.to_device(xh), cos, sin, q, k, v, cache, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    dims = O.dims_of(s)
    qr, rr = O.project(Wd, O.decode_tensor(s.act, xh.data), np.arange(T) + p0, dims)
    Kr, Vr = O.expand_kv(Wd, rr, dims)
    assert_close(torch_io.to_f64(q), qr, s.act, "q")
    assert_close(torch_io.to_f64(k), Kr, s.act, "k")
    assert_close(torch_io.to_f64(v), Vr, s.act, "v")
    flat = torch_io.to_f64(cache).reshape(-1, s.row)
    assert_close(flat[slots], rr, s.act, "cache rows")


@pytest.mark.parametrize("w", [YN_DECODE, YN_DECODE_V3], ids=lambda w: w.name)
def test_decode_step_yarn_input_norm(w):
    """Front end (input norm, YaRN tables built from context_lens on the device), absorbed
    attention with YaRN's score scale over a cache holding the history, and o_proj."""
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[decode+yarn+norm] {w.name} B={w.B}", flush=True)
    host = synth.make_weights(w)
    Wd, dw = O.decode_weights(host), device_weights(host)
    cfg = _cfg(s)
    dims = O.dims_of(s)
    assert abs(cfg.softmax_scale - dims["softmax_scale"]) < 1e-7 * dims["softmax_scale"]
    ctx = YN_CTX[w.number]
    pg = synth.make_paging(w.number, ctx, s.block_size)
    cache_h = np.zeros((pg.n_blocks, s.block_size, s.row), np.uint16)
    hist = []
    for b, n in enumerate(ctx):
        rows = synth.history_rows(w, b, int(n)).data
        synth.fill_cache(cache_h, pg, b, rows)
        hist.append(O.decode_tensor(s.act, rows[:n - 1]))
    cache = torch_io.to_device(synth.Tensor(synth.BF16, cache_h)).view(pg.n_blocks, 1, s.block_size, s.row)
    cl = torch.from_numpy(ctx).cuda()
    inv = mla.mla_rope_inv_freq(_lib_rope(s), s.qk_rope)
    cos, sin = mla.mla_rope_tables(cl, w.B, s.qk_rope, inv, pos_offset=-1)
    xh = synth.make_x(w, w.B, "x.decode")
    q = torch_io.empty_act(s.act, (w.B, s.n_heads, s.qk_head))
    o = torch_io.empty_act(s.act, (w.B, s.n_heads, s.v_dim))
    y = torch_io.empty_act(s.act, (w.B, s.hidden))
    mla.mla_decode_qkv_and_scatter(cfg, dw, torch_io.to_device(xh), cos, sin, cache,
                                   torch.from_numpy(synth.decode_slot_mapping(pg)).cuda(), q)
    mla.mla_decode_attn_absorbed(cfg, dw, q, cache, torch.from_numpy(pg.block_table).cuda(), cl, o)
    mla.mla_out_proj(cfg, dw, o, y)
    torch.cuda.synchronize()
    ref = O.mla_decode(Wd, O.decode_tensor(s.act, xh.data), hist, dims)
    assert_close(torch_io.to_f64(q), ref["q"], s.act, "q")
    assert_close(torch_io.to_f64(o), ref["o"], s.act, "o")
    assert_close(torch_io.to_f64(y), ref["y"], s.act, "y")


def test_prefill_attn_yarn_scale():
    need_gpu()
    import head_latent_attention_amd as mla
    w = YN_PREFILL
    s, T = w.shape, 300
    print(f"[prefill_attn+yarn scale] {w.name} T={T}", flush=True)
    cfg = _cfg(s)
    qh = synth.make_normal(w, "attn.q", (T, s.n_heads, s.qk_head))
    kh = synth.make_normal(w, "attn.k", (T, s.n_heads, s.qk_head))
    vh = synth.make_normal(w, "attn.v", (T, s.n_heads, s.v_dim))
    o = torch_io.empty_act(s.act, (T, s.n_heads, s.v_dim))
    mla.mla_prefill_attn(cfg, torch_io.to_device(qh), torch_io.to_device(kh), torch_io.to_device(vh), o)
    torch.cuda.synchronize()
    q64, k64, v64 = (O.decode_tensor(s.act, t.data) for t in (qh, kh, vh))
    ref = O.attention(q64, k64, v64, O.dims_of(s)["softmax_scale"], np.arange(T))
    assert_close(torch_io.to_f64(o), ref, s.act, "o")
