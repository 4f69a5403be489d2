"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before touching HIP."""
import ctypes
import os
import re

import pytest

import head_latent_attention_amd as mla
from head_latent_attention_amd import binding as B

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "mla.h")
PEAKS_HEADER = os.path.join(INCLUDE, "mla_peaks.h")


def _declared(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = mla.load()
    names = _declared()
    assert set(names) == set(B.SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n


def test_headers_are_all_covered():
    assert sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h")) == ["mla.h", "mla_peaks.h"]


def test_peak_probes_exported_and_validate():
    """The measurement probes' library exports what its header declares and refuses bad
    arguments before any launch."""
    from head_latent_attention_amd import measure as M
    lib = M.load()
    names = _declared(PEAKS_HEADER)
    assert set(names) == set(M.SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mla_peak_read(None, 16, 1, 1, None) == -1
    assert lib.mla_peak_read(16, 24, 1, 1, None) == -1           # not a multiple of 16
    assert lib.mla_peak_read(8, 16, 1, 1, None) == -1            # misaligned
    assert lib.mla_peak_copy(0x1000, 0x1010, 64, 1, None) == -1  # overlapping
    assert lib.mla_peak_mfma_bf16(8, 1, 1.0, 16, 1, 256, None) == -1
    assert lib.mla_peak_mfma_bf16(16, 1, 1.0, 16, 1, 128, None) == -1
    assert lib.mla_peak_mfma_bf16(32, 0, 1.0, 16, 1, 256, None) == -1


def _cfg(**kw):
    c = dict(hidden=256, n_heads=4, q_lora_rank=64, kv_lora_rank=64, qk_nope=32, qk_rope=16, v_dim=32,
             act="f32", weight="f32", block_size=16)
    c.update(kw)
    return mla.config(**c)


def test_status_strings():
    lib = mla.load()
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(-3) == b"workspace too small"


def test_workspace_size_validation():
    lib = mla.load()
    good = _cfg()
    for fn in range(5):
        assert B.workspace_size(good, fn, 8, 64) > 0 or fn == B.FN_PREFILL_ATTN
    assert B.workspace_size(good, 7, 8, 64) == 0
    assert B.workspace_size(good, B.FN_DECODE_ATTN, 8, 0) == 0
    assert B.workspace_size(_cfg(qk_rope=15), 0, 8) == 0
    assert B.workspace_size(_cfg(act="f32", weight="bf16"), 0, 8) == 0
    assert B.workspace_size(good, 0, 0) == 0


def _call_decode_attn(cfg, ws_bytes=1 << 30, q=1, kv=1, bt=1, ctx=1, o=1, B_=1, max_blocks=1, n_blocks=1,
                      wkv_b=1):
    lib = mla.load()
    W = B.MlaWeights()
    W.wkv_b = B.MlaWeight(wkv_b, None)
    return lib.mla_decode_attn_absorbed(ctypes.byref(cfg), ctypes.byref(W), q, B_, kv, n_blocks, bt, max_blocks,
                                        ctx, o, 1, ws_bytes, None)


def test_invalid_arguments_fail_before_launch():
    cfg = _cfg()
    assert _call_decode_attn(cfg, q=None) == -1
    assert _call_decode_attn(cfg, B_=0) == -1
    assert _call_decode_attn(cfg, max_blocks=0) == -1
    assert _call_decode_attn(cfg, wkv_b=None) == -1
    assert _call_decode_attn(_cfg(qk_rope=7)) == -1
    assert _call_decode_attn(_cfg(act="bf16", weight="f32")) == -2
    assert _call_decode_attn(_cfg(weight="fp8", act="bf16"), wkv_b=1) == -1  # fp8 weight without scales
    assert _call_decode_attn(cfg, ws_bytes=16) == -3
    lib = mla.load()
    assert lib.mla_prefill_attn(ctypes.byref(cfg), 1, 1, 1, 0, 1, 1, 1 << 20, None) == -1
    assert lib.mla_out_proj(ctypes.byref(cfg), None, 1, 4, 1, 1, 1 << 20, None) == -1
    W = B.MlaWeights()
    assert lib.mla_qkv_prefill(ctypes.byref(cfg), ctypes.byref(W), 1, 4, 1, 1, 1, 1, 1, None, None, 0, 1,
                               1 << 20, None) == -1
    assert lib.mla_decode_qkv_and_scatter(None, ctypes.byref(W), 1, 4, 1, 1, 1, 1, 1, 1, 1, 1 << 20, None) == -1


def test_rope_entry_points_validate_before_launch():
    lib = mla.load()
    r = mla.rope(factor=40.0)
    assert lib.mla_rope_inv_freq(None, 64, 1, None) == -1
    assert lib.mla_rope_inv_freq(ctypes.byref(r), 63, 1, None) == -1
    assert lib.mla_rope_inv_freq(ctypes.byref(r), 64, None, None) == -1
    assert lib.mla_rope_inv_freq(ctypes.byref(mla.rope(theta=1.0)), 64, 1, None) == -1
    assert lib.mla_rope_inv_freq(ctypes.byref(mla.rope(factor=4.0, original_max_position=0)), 64, 1, None) == -1
    assert lib.mla_rope_inv_freq(ctypes.byref(mla.rope(factor=4.0, beta_fast=1.0, beta_slow=2.0)), 64, 1, None) == -1
    assert lib.mla_rope_tables(0, 64, None, 0, None, 1, 1, None) == -1
    assert lib.mla_rope_tables(4, 7, None, 0, None, 1, 1, None) == -1
    assert lib.mla_rope_tables(4, 64, None, 0, None, None, 1, None) == -1


def test_rope_score_scale_host_function():
    """Host-side score scale against the oracle's (1/sqrt(dqk) times YaRN's magnitude squared)."""
    from oracle import mla_oracle as O
    lib = mla.load()
    assert lib.mla_rope_score_scale(None, 128, 64) == pytest.approx(O.softmax_scale(128, 64), rel=1e-15)
    for f, m in [(40.0, 1.0), (4.0, 0.707), (1.0, 1.0), (0.5, 1.0)]:
        r = mla.rope(factor=f, mscale_all_dim=m)
        assert lib.mla_rope_score_scale(ctypes.byref(r), 128, 64) == pytest.approx(O.softmax_scale(128, 64, f, m),
                                                                                   rel=1e-14)
    assert lib.mla_rope_score_scale(None, 128, 0) == 0.0
    cfg = mla.config(7168, 128, 1536, 512, 128, 64, 128, rope=mla.rope(factor=40.0))
    assert cfg.softmax_scale == pytest.approx(O.softmax_scale(128, 64, 40.0, 1.0), rel=1e-7)


def test_prefill_attn_paged_validation():
    lib = mla.load()
    cfg = _cfg()
    W = B.MlaWeights()
    W.wkv_b = B.MlaWeight(1, None)

    def call(T=4, prefix=0, max_blocks=2, q=1, bt=1, ws_bytes=1 << 30, w=W):
        return lib.mla_prefill_attn_paged(ctypes.byref(cfg), ctypes.byref(w), q, T, 1, 4, bt, max_blocks, prefix, 1,
                                          1, ws_bytes, None)
    assert call(T=0) == -1
    assert call(prefix=-1) == -1
    assert call(q=None) == -1
    assert call(bt=None) == -1
    assert call(prefix=30, T=3) == -1            # prefix + T beyond max_blocks * bs = 32
    assert call(w=B.MlaWeights()) == -1          # wkv_b missing
    assert call(ws_bytes=8) == -3
    assert B.workspace_size(cfg, B.FN_PREFILL_ATTN_PAGED, 8, 64) > B.workspace_size(cfg, B.FN_DECODE_ATTN, 8, 64)
    assert B.workspace_size(cfg, B.FN_PREFILL_ATTN_PAGED, 8, 0) == 0


def test_act_quant_config_and_quantize_validation():
    lib = mla.load()
    # act_quant needs bf16 activations with fp8 weights, and is 0 or 1
    assert B.workspace_size(_cfg(act="bf16", weight="fp8", act_quant=True), 0, 8) > 0
    assert B.workspace_size(_cfg(act="bf16", weight="bf16", act_quant=True), 0, 8) == 0
    bad = _cfg(act="bf16", weight="fp8")
    bad.act_quant = 2
    assert B.workspace_size(bad, 0, 8) == 0
    assert _call_decode_attn(_cfg(act="bf16", weight="bf16", act_quant=True)) == -2
    # quantised activations take workspace of their own
    assert B.workspace_size(_cfg(act="bf16", weight="fp8", act_quant=True), B.FN_OUT_PROJ, 8) > \
        B.workspace_size(_cfg(act="bf16", weight="fp8"), B.FN_OUT_PROJ, 8)
    assert lib.mla_quantize_fp8(None, 4, 128, 128, 1, 1, None) == -1
    assert lib.mla_quantize_fp8(1, 0, 128, 128, 1, 1, None) == -1
    assert lib.mla_quantize_fp8(1, 4, 128, 100, 1, 1, None) == -1   # row stride below K
    assert lib.mla_quantize_fp8(1, 4, 128, 128, None, 1, None) == -1


# ---- the Python binding's argument checks (no GPU: every rejection happens before a pointer
# is taken or the library is called)
import torch  # noqa: E402


def _host_weights(cfg, **override):
    """A Weights holder over host tensors (its device struct is never built)."""
    w = B.Weights.__new__(B.Weights)
    wdt = torch.bfloat16 if cfg.weight_dtype == B.MLA_BF16 else torch.float32
    w.tensors = {n: torch.zeros(s, dtype=torch.float32 if n.endswith("_norm_w") else wdt)
                 for n, s in B.weight_shapes(cfg).items() if n != "input_norm_w"}
    w.scales = {}
    w.tensors.update(override)
    return w


def _bf16_cfg():
    return mla.config(256, 4, 64, 64, 32, 16, 32, act="bf16", weight="bf16", block_size=16, softmax_scale=0.1)


def test_binding_rejects_int64_indices():
    cfg = _bf16_cfg()
    Bq, H = 3, cfg.n_heads
    q = torch.zeros(Bq, H, 48, dtype=torch.bfloat16)
    o = torch.zeros(Bq, H, 32, dtype=torch.bfloat16)
    cache = torch.zeros(4, 1, 16, 80, dtype=torch.bfloat16)
    bt32 = torch.zeros(Bq, 4, dtype=torch.int32)
    ctx32 = torch.ones(Bq, dtype=torch.int32)
    w = _host_weights(cfg)
    with pytest.raises(B.MlaError, match="block_table must have dtype torch.int32"):
        B.mla_decode_attn_absorbed(cfg, w, q, cache, bt32.long(), ctx32, o)
    with pytest.raises(B.MlaError, match="context_lens must have dtype torch.int32"):
        B.mla_decode_attn_absorbed(cfg, w, q, cache, bt32, ctx32.long(), o)
    x = torch.zeros(Bq, cfg.hidden, dtype=torch.bfloat16)
    cs = torch.zeros(Bq, 8, dtype=torch.float32)
    with pytest.raises(B.MlaError, match="slot_mapping must have dtype torch.int32"):
        B.mla_decode_qkv_and_scatter(cfg, w, x, cs, cs, cache, torch.zeros(Bq, dtype=torch.int64), q)
    with pytest.raises(B.MlaError, match="block_table must have dtype torch.int32"):
        B.mla_prefill_attn_paged(cfg, w, q, cache, torch.zeros(4, dtype=torch.int64), 0, o)


def test_binding_rejects_wrong_act_dtype_and_sizes():
    cfg = _bf16_cfg()
    w = _host_weights(cfg)
    T, H = 5, cfg.n_heads
    q = torch.zeros(T, H, 48, dtype=torch.bfloat16)
    k = torch.zeros(T, H, 48, dtype=torch.bfloat16)
    v = torch.zeros(T, H, 32, dtype=torch.bfloat16)
    with pytest.raises(B.MlaError, match="q must have dtype torch.bfloat16"):
        B.mla_prefill_attn(cfg, q.float(), k, v, v.clone())
    with pytest.raises(B.MlaError, match="o must have 640 elements"):
        B.mla_prefill_attn(cfg, q, k, v, v[:4].clone())
    with pytest.raises(B.MlaError, match="y must have shape"):
        B.mla_out_proj(cfg, w, v.reshape(T, -1), torch.zeros(T, 255, dtype=torch.bfloat16))
    x = torch.zeros(T, cfg.hidden, dtype=torch.bfloat16)
    cs = torch.zeros(T, 8, dtype=torch.float32)
    with pytest.raises(B.MlaError, match="x must have dtype torch.bfloat16"):
        B.mla_qkv_prefill(cfg, w, x.float(), cs, cs, q, k, v)
    with pytest.raises(B.MlaError, match="cos must have 40 elements"):
        B.mla_qkv_prefill(cfg, w, x, cs[:4], cs, q, k, v)
    # the cache must be [n_blocks, 1, block_size, kv_lora + rope]: a flat [slots, row] view is refused
    bt = torch.zeros(T, 2, dtype=torch.int32)
    ctx = torch.ones(T, dtype=torch.int32)
    flat = torch.zeros(64, 80, dtype=torch.bfloat16)
    with pytest.raises(B.MlaError, match="kv_cache must have shape"):
        B.mla_decode_attn_absorbed(cfg, w, q, flat, bt, ctx, v)
    with pytest.raises(B.MlaError, match="kv_cache must have shape"):
        B.mla_decode_attn_absorbed(cfg, w, q, torch.zeros(4, 1, 32, 80, dtype=torch.bfloat16), bt, ctx, v)


def test_binding_rejects_mismatched_weights():
    cfg = _bf16_cfg()
    T, H = 5, cfg.n_heads
    v = torch.zeros(T, H, 32, dtype=torch.bfloat16)
    y = torch.zeros(T, cfg.hidden, dtype=torch.bfloat16)
    with pytest.raises(B.MlaError, match="wo must have shape"):
        B.mla_out_proj(cfg, _host_weights(cfg, wo=torch.zeros(128, 255, dtype=torch.bfloat16)), v, y)
    with pytest.raises(B.MlaError, match="wo must have dtype"):
        B.mla_out_proj(cfg, _host_weights(cfg, wo=torch.zeros(128, 256, dtype=torch.float32)), v, y)
    cfg8 = mla.config(256, 4, 64, 64, 32, 16, 32, act="bf16", weight="fp8", block_size=16, softmax_scale=0.1)
    w8 = _host_weights(cfg8, wo=torch.zeros(128, 256, dtype=torch.uint8))
    with pytest.raises(B.MlaError, match="wo scale is required"):
        B.mla_out_proj(cfg8, w8, v, y)


def test_noalloc_entry_point_validates_before_launch():
    """The no-alloc decode attention refuses bad arguments and batches beyond its static scratch
    with a status, before touching HIP."""
    lib = mla.load()
    cfg = mla.config(7168, 128, 1536, 512, 128, 64, 128, softmax_scale=0.072)
    W = B.MlaWeights()
    W.wkv_b = B.MlaWeight(1, None)

    def call(Bn=4, max_blocks=8, q=1, w=W):
        return lib.mla_decode_attn_absorbed_noalloc(ctypes.byref(cfg), ctypes.byref(w), q, Bn, 1, 64, 1, max_blocks,
                                                    1, 1, None)
    assert call(Bn=0) == -1
    assert call(q=None) == -1
    assert call(w=B.MlaWeights()) == -1
    assert B.workspace_size(cfg, B.FN_DECODE_ATTN, 130, 512) > B.NOALLOC_SCRATCH_BYTES
    assert call(Bn=130) == -3
    assert B.workspace_size(cfg, B.FN_DECODE_ATTN, 119, 1 << 20) <= B.NOALLOC_SCRATCH_BYTES
