"""mla_decode_attn_absorbed_noalloc (static scratch, no workspace) against mla_decode_attn_absorbed
(caller workspace): the same kernels on the same inputs must give the same output bit for bit,
on two calls in a row, the second with a smaller batch than the first (the scratch keeps the
first call's contents; nothing in it may leak into the second)."""
import numpy as np
import pytest
import torch

import synth
from synth import torch_io
from helpers import device_weights, lib_config, need_gpu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
# the V3 decode batch (B = 64, contexts 1024..8192), then six sequences with edge contexts
CALLS = [(W[3], None), (synth.custom(W[3], 120, "noalloc-edge-b6", B=6), np.array([1, 63, 64, 65, 200, 1000], np.int32))]


def _inputs(w, ctx):
    s = w.shape
    if ctx is None:
        ctx = synth.context_lengths(w)
    pg = synth.make_paging(w.number, ctx, s.block_size)
    cache = torch.empty((pg.n_blocks, 1, s.block_size, s.row), dtype=torch.bfloat16, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(700 + w.number)
    flat = cache.view(-1, s.row)
    vals = torch.randn(flat.shape, generator=gen, device="cuda", dtype=torch.float32)
    vals[:, s.kv_lora_rank:] *= 0.02 * float(np.sqrt(s.hidden))
    flat.copy_(vals.to(torch.bfloat16))
    q = torch_io.to_device(synth.make_normal(w, "decode.q", (w.B, s.n_heads, s.qk_head), std=0.8))
    return ctx, pg, cache, q


def test_noalloc_matches_workspace_entry_point_twice():
    need_gpu()
    import head_latent_attention_amd as mla
    w0 = CALLS[0][0]
    dw = device_weights(synth.make_weights(w0))  # the V3 weights serve both calls
    cfg = lib_config(w0.shape)
    for w, ctx in CALLS:
        s = w.shape
        ctx, pg, cache, q = _inputs(w, ctx)
        bt = torch.from_numpy(pg.block_table).cuda()
        cl = torch.from_numpy(ctx).cuda()
        print(f"[noalloc] B={w.B} contexts {int(ctx.min())}..{int(ctx.max())}", flush=True)
        o_ws = torch.full((w.B, s.n_heads, s.v_dim), 3.0, dtype=torch.bfloat16, device="cuda")
        o_na = torch.full((w.B, s.n_heads, s.v_dim), 5.0, dtype=torch.bfloat16, device="cuda")
        mla.mla_decode_attn_absorbed(cfg, dw, q, cache, bt, cl, o_ws)
        mla.mla_decode_attn_absorbed_noalloc(cfg, dw, q, cache, bt, cl, o_na)
        torch.cuda.synchronize()
        same = torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
        print(f"  o: {'identical' if same else 'DIFFERENT'} to the workspace entry point", flush=True)
        assert torch.isfinite(o_na.float()).all()
        assert same


def test_noalloc_rejects_batches_beyond_the_scratch():
    """A batch whose workspace need exceeds the static scratch is refused before any launch."""
    need_gpu()
    import head_latent_attention_amd as mla
    from head_latent_attention_amd import binding as B
    w = synth.custom(W[3], 121, "noalloc-b130", B=130, ctx_lo=64, ctx_hi=64)
    s = w.shape
    cfg = lib_config(s)
    assert B.workspace_size(cfg, B.FN_DECODE_ATTN, w.B, 64) > B.NOALLOC_SCRATCH_BYTES
    dw = device_weights(synth.make_weights(W[3]))
    ctx = np.full(w.B, 64, np.int32)
    pg = synth.make_paging(w.number, ctx, s.block_size)
    cache = torch.zeros((pg.n_blocks, 1, s.block_size, s.row), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((w.B, s.n_heads, s.qk_head), dtype=torch.bfloat16, device="cuda")
    o = torch.full((w.B, s.n_heads, s.v_dim), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError, match="workspace"):
        mla.mla_decode_attn_absorbed_noalloc(cfg, dw, q, cache, torch.from_numpy(pg.block_table).cuda(),
                                             torch.from_numpy(ctx).cuda(), o)
    torch.cuda.synchronize()
    assert bool((o.float() == 7.0).all())  # untouched
