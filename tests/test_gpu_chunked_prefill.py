"""GPU parity of chunked prefill over a paged prefix (mla_qkv_prefill without the K/V
expansion writes the chunk's rows, then mla_prefill_attn_paged attends over prefix + chunk)
against the oracle's expanded causal attention of the chunk over the whole sequence."""
import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O
from synth import torch_io
from helpers import assert_close, device_weights, lib_config, need_gpu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CH_TINY = synth.custom(W[1], 140, "chunk-tiny-fp32")
CH_V3 = synth.custom(W[3], 141, "chunk-v3-heads", hidden=1024, q_lora_rank=256)
CH_V3_FULL = synth.custom(W[3], 142, "chunk-v3")
# the same workload in 96- and 32-token cache blocks
CH_V3_BS96 = synth.custom(W[3], 141, "chunk-v3-heads-bs96", hidden=1024, q_lora_rank=256, block_size=96)
CH_V3_BS32 = synth.custom(W[3], 141, "chunk-v3-heads-bs32", hidden=1024, q_lora_rank=256, block_size=32)


def _run_chunk(w, dw, cfg, cache, table, prefix, T, xh):
    """Front end of the chunk (rows scattered at positions prefix..), then paged attention."""
    import head_latent_attention_amd as mla
    s = w.shape
    pos = np.arange(prefix, prefix + T)
    slots = synth.slots_for(table, pos, s.block_size)
    cos, sin = mla.rope_cos_sin(pos, s.qk_rope)
    q = torch_io.empty_act(s.act, (T, s.n_heads, s.qk_head))
    mla.mla_qkv_prefill(cfg, dw, torch_io.to_device(xh), cos, sin, q, None, None, cache,
                        torch.from_numpy(slots).cuda())
    o = torch_io.empty_act(s.act, (T, s.n_heads, s.v_dim))
    mla.mla_prefill_attn_paged(cfg, dw, q, cache, torch.from_numpy(table).cuda(), prefix, o)
    torch.cuda.synchronize()
    return q, o


def test_chunks_after_prefill_tiny_fp32():
    """80 tokens: a 48-token prefill, then chunks of 31 and 1 tokens; every chunk's output
    equals the oracle's causal attention of those tokens over the whole sequence."""
    need_gpu()
    import head_latent_attention_amd as mla
    w = CH_TINY
    s = w.shape
    print(f"[chunk] {w.name}", flush=True)
    host = synth.make_weights(w)
    Wd, dw = O.decode_weights(host), device_weights(host)
    cfg = lib_config(s)
    N = 80
    x = synth.make_x(w, N, "x.chunked")
    n_blocks = 8
    table = synth.shuffled_blocks(w.number, "blocks", n_blocks)[:6].copy()
    cache = torch.zeros((n_blocks, 1, s.block_size, s.row), dtype=torch.float32, device="cuda")
    dims = O.dims_of(s)
    x64 = O.decode_tensor(s.act, x.data)
    qr, rr = O.project(Wd, x64, np.arange(N), dims)
    start = 0
    for T in (48, 31, 1):
        xs = synth.Tensor(x.kind, x.data[start:start + T])
        _, o = _run_chunk(w, dw, cfg, cache, table, start, T, xs)
        ref = O.chunk_attention(Wd, qr[start:start + T], rr[:start], rr[start:start + T], dims)
        assert_close(torch_io.to_f64(o), ref, s.act, f"o of tokens {start}..{start + T - 1}")
        start += T


# (0, 130), (1000, 77) and (64, 1) take the absorbed form; (3000, 300), (600, 400) and (4096, 512)
# the expanded one (more than ~170 queries per cached row), (600, 400) with its expansion through
# the smaller projection kernel (1000 rows)
@pytest.mark.parametrize("w,prefix,T", [(CH_V3, 0, 130), (CH_V3, 1000, 77), (CH_V3, 3000, 300), (CH_V3, 64, 1),
                                        (CH_V3, 600, 400), (CH_V3_FULL, 4096, 512), (CH_V3_BS96, 1000, 77),
                                        (CH_V3_BS96, 3000, 300), (CH_V3_BS32, 600, 400)],
                         ids=lambda c: str(c) if isinstance(c, int) else c.name)
def test_chunk_over_cached_history(w, prefix, T):
    """A chunk of T tokens over `prefix` history rows already in the paged cache (V2/V3 per-head
    dims, the matrix-core path); positions past the chunk's last block are never read."""
    need_gpu()
    s = w.shape
    print(f"[chunk] {w.name} prefix={prefix} T={T}", flush=True)
    host = synth.make_weights(w)
    Wd, dw = O.decode_weights(host), device_weights(host)
    cfg = lib_config(s)
    N = prefix + T
    pg = synth.make_paging(w.number, np.array([N + 70], np.int32), s.block_size)  # spare table entries
    hist = synth.history_rows(w, 0, N).data
    cache_h = np.zeros((pg.n_blocks, s.block_size, s.row), np.uint16)
    synth.fill_cache(cache_h, pg, 0, hist)  # rows past the prefix are overwritten by the chunk
    cache = torch_io.to_device(synth.Tensor(synth.BF16, cache_h)).view(pg.n_blocks, 1, s.block_size, s.row)
    xh = synth.make_x(w, T, f"x.chunk.{prefix}")
    q, o = _run_chunk(w, dw, cfg, cache, pg.block_table[0], prefix, T, xh)
    dims = O.dims_of(s)
    qr, rr = O.project(Wd, O.decode_tensor(s.act, xh.data), np.arange(prefix, N), dims)
    assert_close(torch_io.to_f64(q), qr, s.act, "q")
    ref = O.chunk_attention(Wd, qr, O.decode_tensor(s.act, hist[:prefix]), rr, dims)
    assert_close(torch_io.to_f64(o), ref, s.act, "o")
