"""A whole decode step (front end, absorbed attention, output projection) captured in a
HIP graph and replayed: every replay must reproduce the eager step bit for bit.

The library allocates nothing and clears nothing with memset, so its launches can be
captured; the replays are interleaved with eager work that overwrites the outputs, and
each replay is checked separately."""
import numpy as np
import pytest
import torch

import synth
from synth import torch_io
from helpers import device_weights, lib_config, need_gpu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
GRAPH_DEC = synth.custom(W[3], 106, "graph-decode-h128", B=6)
GRAPH_CTX = np.array([1, 63, 64, 65, 200, 1000], np.int32)


def _setup(w, ctx):
    import head_latent_attention_amd as mla
    s = w.shape
    host = synth.make_weights(w)
    dw = device_weights(host)
    cfg = lib_config(s)
    pg = synth.make_paging(w.number, ctx, s.block_size)
    cache_h = np.zeros((pg.n_blocks, s.block_size, s.row), np.uint16)
    for b, n in enumerate(ctx):
        synth.fill_cache(cache_h, pg, b, synth.history_rows(w, b, int(n)).data)
    cache = torch_io.to_device(synth.Tensor(synth.BF16, cache_h)).view(pg.n_blocks, 1, s.block_size, s.row)
    x = torch_io.to_device(synth.make_x(w, w.B, "x.decode"))
    cos, sin = mla.rope_cos_sin(ctx.astype(np.int64) - 1, s.qk_rope)
    st = dict(cfg=cfg, dw=dw, cache=cache, x=x, cos=cos, sin=sin,
              slot=torch.from_numpy(synth.decode_slot_mapping(pg)).cuda(),
              bt=torch.from_numpy(pg.block_table).cuda(), cl=torch.from_numpy(ctx).cuda(),
              q=torch_io.empty_act(s.act, (w.B, s.n_heads, s.qk_head)),
              o=torch_io.empty_act(s.act, (w.B, s.n_heads, s.v_dim)),
              y=torch_io.empty_act(s.act, (w.B, s.hidden)))
    max_ctx = pg.block_table.shape[1] * s.block_size
    st["ws"] = (mla.workspace(cfg, 2, w.B), mla.workspace(cfg, 3, w.B, max_ctx), mla.workspace(cfg, 4, w.B))
    return st


def _step(st):
    import head_latent_attention_amd as mla
    mla.mla_decode_qkv_and_scatter(st["cfg"], st["dw"], st["x"], st["cos"], st["sin"], st["cache"], st["slot"],
                                   st["q"], ws=st["ws"][0])
    mla.mla_decode_attn_absorbed(st["cfg"], st["dw"], st["q"], st["cache"], st["bt"], st["cl"], st["o"],
                                 ws=st["ws"][1])
    mla.mla_out_proj(st["cfg"], st["dw"], st["o"], st["y"], ws=st["ws"][2])


def test_decode_step_graph_replays():
    need_gpu()
    w = GRAPH_DEC
    print(f"[graph] {w.name} B={w.B}", flush=True)
    st = _setup(w, GRAPH_CTX)
    _step(st)
    torch.cuda.synchronize()
    ref = {k: st[k].clone() for k in ("q", "o", "y", "cache")}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(st)
    torch.cuda.synchronize()
    for r in range(3):
        for k in ("q", "o", "y"):
            st[k].fill_(float(r + 7))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("q", "o", "y", "cache"):
            same = torch.equal(st[k].view(torch.int16), ref[k].view(torch.int16))
            print(f"  replay {r} {k}: {'identical' if same else 'DIFFERENT'}", flush=True)
            assert same, f"replay {r}: {k} differs from the eager step"
