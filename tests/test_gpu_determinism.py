"""Run-to-run determinism at full size: the same inputs give bitwise identical outputs.

The decode step (front end with its cache scatter, absorbed attention, output projection)
mutates the paged cache in place ([NKI-Decode] kv_cache and slot_mapping parameters); run
twice, it must write the same row to the same slot and produce the same q, o and y.  The
prefill chain (projections with their split-K sums, the persistent attention, o_proj) must
likewise reproduce itself exactly: every reduction runs in a fixed order."""
import numpy as np
import pytest
import torch

import synth
from synth import torch_io
from helpers import device_weights, lib_config, need_gpu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _device_cache(w, pg):
    """Rows of the history distribution drawn on the device from one seeded generator."""
    s = w.shape
    cache = torch.empty((pg.n_blocks, 1, s.block_size, s.row), dtype=torch.bfloat16, device="cuda")
    flat = cache.view(-1, s.row)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(500 + w.number)
    for r0 in range(0, flat.shape[0], 1 << 20):
        blk = flat[r0:r0 + (1 << 20)]
        vals = torch.randn(blk.shape, generator=gen, device="cuda", dtype=torch.float32)
        vals[:, s.kv_lora_rank:] *= 0.02 * float(np.sqrt(s.hidden))
        blk.copy_(vals.to(torch.bfloat16))
    return cache


@pytest.mark.parametrize("w", [W[3], W[5]], ids=lambda w: w.name)
def test_decode_step_bitwise_repeatable(w):
    need_gpu()
    import head_latent_attention_amd as mla
    s = w.shape
    print(f"[determinism] {w.name} B={w.B}", flush=True)
    dw = device_weights(synth.make_weights(w))
    cfg = lib_config(s)
    ctx = synth.context_lengths(w)
    pg = synth.make_paging(w.number, ctx, s.block_size)
    cache = _device_cache(w, pg)
    x = torch_io.to_device(synth.make_x(w, w.B, "x.decode"))
    slot = torch.from_numpy(synth.decode_slot_mapping(pg)).cuda()
    bt = torch.from_numpy(pg.block_table).cuda()
    cl = torch.from_numpy(ctx).cuda()
    cos, sin = mla.mla_rope_tables(cl, w.B, s.qk_rope, None, pos_offset=-1)
    max_ctx = pg.block_table.shape[1] * s.block_size
    ws = (mla.workspace(cfg, 2, w.B), mla.workspace(cfg, 3, w.B, max_ctx), mla.workspace(cfg, 4, w.B))
    outs = []
    for run in range(2):
        q = torch.full((w.B, s.n_heads, s.qk_head), float(run + 3), dtype=torch.bfloat16, device="cuda")
        o = torch.full((w.B, s.n_heads, s.v_dim), float(run + 3), dtype=torch.bfloat16, device="cuda")
        y = torch.full((w.B, s.hidden), float(run + 3), dtype=torch.bfloat16, device="cuda")
        for t in ws:
            t.fill_(0x5A + run)  # workspace contents differ between the runs
        mla.mla_decode_qkv_and_scatter(cfg, dw, x, cos, sin, cache, slot, q, ws=ws[0])
        mla.mla_decode_attn_absorbed(cfg, dw, q, cache, bt, cl, o, ws=ws[1])
        mla.mla_out_proj(cfg, dw, o, y, ws=ws[2])
        torch.cuda.synchronize()
        rows = cache.view(-1, s.row)[slot.long()].clone()
        outs.append((q, o, y, rows))
    for name, a, b in zip(("q", "o", "y", "scattered rows"), outs[0], outs[1]):
        same = torch.equal(_bits(a), _bits(b))
        print(f"  {name}: {'identical' if same else 'DIFFERENT'}", flush=True)
        assert same, f"{name} differs between two runs"
    assert torch.isfinite(outs[0][2].float()).all()


def test_prefill_chain_bitwise_repeatable():
    need_gpu()
    import head_latent_attention_amd as mla
    w = W[4]
    s, T = w.shape, w.T
    print(f"[determinism] {w.name} T={T}", flush=True)
    dw = device_weights(synth.make_weights(w))
    cfg = lib_config(s)
    x = torch_io.to_device(synth.make_x(w, T))
    cos, sin = mla.rope_cos_sin(np.arange(T), s.qk_rope)
    n_blocks = -(-T // s.block_size)
    slots = torch.from_numpy(synth.slots_for(synth.shuffled_blocks(w.number, "blocks", n_blocks), np.arange(T),
                                             s.block_size)).cuda()
    outs = []
    for run in range(2):
        cache = torch.full((n_blocks, 1, s.block_size, s.row), float(run + 3), dtype=torch.bfloat16, device="cuda")
        q = torch.empty((T, s.n_heads, s.qk_head), dtype=torch.bfloat16, device="cuda")
        k = torch.empty_like(q)
        v = torch.empty((T, s.n_heads, s.v_dim), dtype=torch.bfloat16, device="cuda")
        o = torch.empty_like(v)
        y = torch.empty((T, s.hidden), dtype=torch.bfloat16, device="cuda")
        mla.mla_qkv_prefill(cfg, dw, x, cos, sin, q, k, v, cache, slots)
        mla.mla_prefill_attn(cfg, q, k, v, o)
        mla.mla_out_proj(cfg, dw, o, y)
        torch.cuda.synchronize()
        outs.append((q, k, v, cache, o, y))
        del q, k, v, cache, o, y
    for name, a, b in zip(("q", "k", "v", "cache", "o", "y"), outs[0], outs[1]):
        same = torch.equal(_bits(a), _bits(b))
        print(f"  {name}: {'identical' if same else 'DIFFERENT'}", flush=True)
        assert same, f"{name} differs between two runs"
