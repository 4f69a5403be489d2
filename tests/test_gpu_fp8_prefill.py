"""GPU parity of the fp8 projections with MX fp8 activations (config act_quant): the
quantisation decision bit for bit, then every projection entry point against the oracle
that quantises the same activations at the same places.

Projections of more than 1024 rows run on the fp8 matrix-core kernel; smaller ones take the
dequantised values through the bf16 kernels; both must match the same oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from synth import torch_io
from helpers import assert_close, device_weights, lib_config, need_gpu, sentinel_cache

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
FP8_SMALL = synth.custom(W[4], 150, "fp8-aq-prefill-small", hidden=1024, n_heads=16, q_lora_rank=256, weight="fp8",
                         act_quant=True, T=1300)
FP8_RAGGED = synth.custom(W[4], 151, "fp8-aq-prefill-ragged", hidden=1024, n_heads=16, q_lora_rank=256,
                          weight="fp8", act_quant=True, T=300)
FP8_C4 = synth.custom(W[4], 152, "fp8-aq-prefill-8192", weight="fp8", act_quant=True)
FP8_DEC = synth.custom(W[5], 153, "fp8-aq-decode", act_quant=True, B=6)

_cache = {}


def _weights(w):
    if w.number not in _cache:
        _cache.clear()
        host = synth.make_weights(w)
        _cache[w.number] = (host, O.decode_weights(host), device_weights(host))
    return _cache[w.number]


def _rows(T, n=12):
    r = np.random.default_rng(0)
    return np.array(sorted({0, 1, 127, 128, 255, 256, T // 2, T - 1} | set(r.integers(0, T, n).tolist())))


@pytest.mark.parametrize("M,K", [(1, 128), (37, 300), (300, 1024), (64, 7168), (2048, 16384)])
def test_quantize_fp8_bit_exact(M, K):
    """Codes and exponents of the device quantiser equal the oracle's on the same bf16 rows:
    mixed magnitudes per row (including 0, subnormal-range and large groups) and ragged K."""
    need_gpu()
    import head_latent_attention_amd as mla
    print(f"[quantize] M={M} K={K}", flush=True)
    r = synth.rng(7, f"quant.{M}.{K}")
    mag = 2.0 ** r.integers(-30, 20, (M, 1))
    x = (r.standard_normal((M, K)) * mag).astype(np.float32)
    x[M // 2, :] = 0.0
    if K > 200:
        x[0, 128:200] = 0.0
        x[0, 5] = 1e-38                                   # group of tiny values
    xt = synth.encode(x, "bf16")
    codes, exps = mla.mla_quantize_fp8(torch_io.to_device(xt))
    torch.cuda.synchronize()
    oc, oe, _ = O.quantize_mx_fp8(O.decode_tensor("bf16", xt.data))
    got_e = exps.cpu().numpy().astype(np.int64) - 127
    assert (got_e == oe.T).all(), np.argwhere(got_e != oe.T)[:5]
    gc = codes.cpu().numpy()
    diff = np.argwhere(gc != oc)
    assert len(diff) == 0, (len(diff), diff[:5], gc[tuple(diff[0])], oc[tuple(diff[0])])


@pytest.mark.parametrize("w", [FP8_SMALL, FP8_RAGGED, FP8_C4], ids=lambda w: w.name)
def test_qkv_prefill_fp8(w):
    need_gpu()
    import head_latent_attention_amd as mla
    s, T = w.shape, w.T
    print(f"[qkv_prefill fp8] {w.name} T={T}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    xh = synth.make_x(w, T)
    n_blocks = -(-T // s.block_size) + 3
    slots = synth.slots_for(synth.shuffled_blocks(w.number, "blocks", n_blocks), np.arange(T), s.block_size)
    cache = sentinel_cache(s, n_blocks)
    cos, sin = mla.rope_cos_sin(np.arange(T), s.qk_rope)
    q = torch_io.empty_act(s.act, (T, s.n_heads, s.qk_head))
    k = torch_io.empty_act(s.act, (T, s.n_heads, s.qk_head))
    v = torch_io.empty_act(s.act, (T, s.n_heads, s.v_dim))
    mla.mla_qkv_prefill(cfg, dw, torch_io.to_device(xh), cos, sin, q, k, v, cache, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    dims = O.dims_of(s)
    assert dims["act_quant"]
    x64 = O.decode_tensor(s.act, xh.data)
    rows = _rows(T) if T > 1000 else np.arange(T)
    qr, rr = O.project(Wd, x64[rows], rows, dims)
    Kr, Vr = O.expand_kv(Wd, rr, dims)
    assert_close(torch_io.to_f64(q)[rows], qr, s.act, "q", rows)
    assert_close(torch_io.to_f64(k)[rows], Kr, s.act, "k", rows)
    assert_close(torch_io.to_f64(v)[rows], Vr, s.act, "v", rows)
    flat = torch_io.to_f64(cache).reshape(-1, s.row)
    assert_close(flat[slots[rows]], rr, s.act, "cache rows", rows)


@pytest.mark.parametrize("w,M", [(FP8_SMALL, 1300), (FP8_SMALL, 64), (FP8_C4, 8192)],
                         ids=lambda c: str(c) if isinstance(c, int) else c.name)
def test_out_proj_fp8(w, M):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[out_proj fp8] {w.name} M={M}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    oh = synth.make_normal(w, f"oproj.o.{M}", (M, s.n_heads * s.v_dim), std=0.5)
    y = torch_io.empty_act(s.act, (M, s.hidden))
    mla.mla_out_proj(cfg, dw, torch_io.to_device(oh), y)
    torch.cuda.synchronize()
    rows = _rows(M) if M > 1000 else np.arange(M)
    ref = O.out_proj(Wd, O.decode_tensor(s.act, oh.data)[rows], O.dims_of(s))
    assert_close(torch_io.to_f64(y)[rows], ref, s.act, "y", rows)


def test_decode_front_end_fp8():
    """act_quant also governs the decode projections (quantised, dequantised, bf16 kernels)."""
    need_gpu()
    import head_latent_attention_amd as mla
    w = FP8_DEC
    s = w.shape
    print(f"[decode qkv fp8] {w.name}", flush=True)
    host, Wd, dw = _weights(w)
    cfg = lib_config(s)
    ctx = np.array([1, 63, 64, 65, 200, 1000], np.int32)
    pg = synth.make_paging(w.number, ctx, s.block_size)
    slots = synth.decode_slot_mapping(pg)
    cache = sentinel_cache(s, pg.n_blocks)
    xh = synth.make_x(w, w.B, "x.decode")
    pos = ctx.astype(np.int64) - 1
    cos, sin = mla.rope_cos_sin(pos, s.qk_rope)
    q = torch_io.empty_act(s.act, (w.B, s.n_heads, s.qk_head))
    mla.mla_decode_qkv_and_scatter(cfg, dw, torch_io.to_device(xh), cos, sin, cache, torch.from_numpy(slots).cuda(), q)
    torch.cuda.synchronize()
    qr, rr = O.project(Wd, O.decode_tensor(s.act, xh.data), pos, O.dims_of(s))
    assert_close(torch_io.to_f64(q), qr, s.act, "q")
    got_rows = torch_io.to_f64(cache.view(-1, s.row)[torch.from_numpy(slots.astype(np.int64)).cuda()])
    assert_close(got_rows, rr, s.act, "cache rows")


def test_non_power_of_two_weight_scale_poisons_its_block():
    """A weight block scale that is not a power of two cannot be applied by the fp8 matrix op:
    the output columns of that block come out NaN, every other column stays finite."""
    need_gpu()
    import head_latent_attention_amd as mla
    w = FP8_SMALL
    s = w.shape
    print("[fp8 scale check]", flush=True)
    host, Wd, dw = _weights(w)
    sc = dw.scales["wo"].clone()
    sc[3, 2] = sc[3, 2] * 1.5                         # row block 3, column block 2 (columns 256..383)
    dw2 = mla.Weights(dw.tensors, dict(dw.scales, wo=sc))
    cfg = lib_config(s)
    M = 1300
    oh = synth.make_normal(w, "oproj.o.scale", (M, s.n_heads * s.v_dim), std=0.5)
    y = torch_io.empty_act(s.act, (M, s.hidden))
    mla.mla_out_proj(cfg, dw2, torch_io.to_device(oh), y)
    torch.cuda.synchronize()
    nan = torch.isnan(y.float()).cpu().numpy()
    assert nan[:, 256:384].all() and not nan[:, :256].any() and not nan[:, 384:].any()
