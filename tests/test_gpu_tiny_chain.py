"""Tiny fp32 MLA layer end to end on the GPU: causal prefill of 64 tokens, then 16
decode steps through the paged cache (block_size 16, shuffled block table),
every output and every cache row compared with the float64 oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from synth import torch_io
from helpers import assert_close, device_weights, lib_config, need_gpu, sentinel_cache

pytestmark = pytest.mark.gpu


def test_tiny_prefill_then_decode():
    need_gpu()
    import head_latent_attention_amd as mla
    w = synth.WORKLOADS[1]
    s = w.shape
    kind = s.act
    print(f"[tiny chain] T={w.T} steps={w.decode_steps}", flush=True)
    host_w = synth.make_weights(w)
    W = O.decode_weights(host_w)
    dims = O.dims_of(s)
    dw = device_weights(host_w)
    cfg = lib_config(s)
    total = w.T + w.decode_steps
    pg = synth.make_paging(w.number, np.array([total]), s.block_size, spare=3)
    assert pg.n_blocks == 8
    bt = pg.block_table[0]
    cache = sentinel_cache(s, pg.n_blocks)
    sentinel_bits = torch_io.bits(cache).reshape(-1, s.row)[0, 0]

    # ---- prefill
    xh = synth.make_x(w, w.T, "x.prefill")
    x = torch_io.to_device(xh)
    slots = synth.slots_for(bt, np.arange(w.T), s.block_size)
    cos, sin = mla.rope_cos_sin(np.arange(w.T), s.qk_rope)
    q = torch_io.empty_act(kind, (w.T, s.n_heads, s.qk_head))
    k = torch_io.empty_act(kind, (w.T, s.n_heads, s.qk_head))
    v = torch_io.empty_act(kind, (w.T, s.n_heads, s.v_dim))
    o = torch_io.empty_act(kind, (w.T, s.n_heads, s.v_dim))
    y = torch_io.empty_act(kind, (w.T, s.hidden))
    mla.mla_qkv_prefill(cfg, dw, x, cos, sin, q, k, v, cache, torch.from_numpy(slots).cuda())
    mla.mla_prefill_attn(cfg, q, k, v, o)
    mla.mla_out_proj(cfg, dw, o, y)
    torch.cuda.synchronize()
    ref = O.mla_prefill(W, O.decode_tensor(kind, xh.data), dims)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("y", y)):
        assert_close(torch_io.to_f64(t), ref[name], kind, f"prefill {name}")
    flat = torch_io.to_f64(cache).reshape(-1, s.row)
    assert_close(flat[slots], ref["rows"], kind, "prefill cache rows")
    hist = list(ref["rows"])

    # ---- decode steps
    xd = synth.make_x(w, w.decode_steps, "x.decode")
    xdev = torch_io.to_device(xd)
    written = set(int(v) for v in slots)
    for step in range(w.decode_steps):
        pos = w.T + step
        slot = synth.slots_for(bt, np.array([pos]), s.block_size)
        cos, sin = mla.rope_cos_sin(np.array([pos]), s.qk_rope)
        qd = torch_io.empty_act(kind, (1, s.n_heads, s.qk_head))
        od = torch_io.empty_act(kind, (1, s.n_heads, s.v_dim))
        yd = torch_io.empty_act(kind, (1, s.hidden))
        mla.mla_decode_qkv_and_scatter(cfg, dw, xdev[step:step + 1].contiguous(), cos, sin, cache,
                                       torch.from_numpy(slot).cuda(), qd)
        bt_dev = torch.from_numpy(pg.block_table).cuda()
        ctx = torch.tensor([pos + 1], dtype=torch.int32, device="cuda")
        mla.mla_decode_attn_absorbed(cfg, dw, qd, cache, bt_dev, ctx, od)
        mla.mla_out_proj(cfg, dw, od, yd)
        torch.cuda.synchronize()
        r = O.mla_decode(W, O.decode_tensor(kind, xd.data[step:step + 1]), [np.array(hist)], dims)
        assert_close(torch_io.to_f64(qd), r["q"], kind, f"step {step} q")
        assert_close(torch_io.to_f64(od), r["o"], kind, f"step {step} o")
        assert_close(torch_io.to_f64(yd), r["y"], kind, f"step {step} y")
        flat = torch_io.to_f64(cache).reshape(-1, s.row)
        assert_close(flat[slot[0]], r["rows"][0], kind, f"step {step} cache row")
        hist.append(r["rows"][0])
        written.add(int(slot[0]))
    # placement is exact: every slot not written still holds the sentinel bits
    b = torch_io.bits(cache).reshape(-1, s.row)
    untouched = np.array(sorted(set(range(b.shape[0])) - written))
    assert (b[untouched] == sentinel_bits).all()
    assert len(written) == total
