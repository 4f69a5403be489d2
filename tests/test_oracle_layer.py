"""Whole-layer pins of the oracle: pure-Python brute force on tiny shapes, the
absorption identity, and decode/prefill consistency."""
import math

import numpy as np
import pytest

import synth
from oracle import mla_oracle as O


def _tiny_weights(seed, D, H, Lq, Lkv, dn, dr, dv, input_norm=False):
    r = synth.rng(seed, "tiny")
    W = {
        "wq_b": r.standard_normal((Lq or D, H * (dn + dr))) * 0.3,
        "wkv_a": r.standard_normal((D, Lkv + dr)) * 0.3,
        "wkv_b": r.standard_normal((Lkv, H * (dn + dv))) * 0.3,
        "wo": r.standard_normal((H * dv, D)) * 0.3,
        "kv_norm_w": 1 + 0.1 * r.standard_normal(Lkv),
    }
    if Lq:
        W["wq_a"] = r.standard_normal((D, Lq)) * 0.3
        W["q_norm_w"] = 1 + 0.1 * r.standard_normal(Lq)
    if input_norm:
        W["input_norm_w"] = 1 + 0.1 * r.standard_normal(D)
    dims = dict(hidden=D, n_heads=H, q_lora_rank=Lq, kv_lora_rank=Lkv, qk_nope=dn, qk_rope=dr,
                v_dim=dv, norm_eps=1e-6, rope_theta=10000.0, softmax_scale=1 / math.sqrt(dn + dr))
    return W, dims


def _rope_pair_loops(vec, pos, theta=10000.0, inv_freq=None):
    dr = len(vec)
    out = list(vec)
    for i in range(dr // 2):
        a = pos * (theta ** (-2.0 * i / dr) if inv_freq is None else inv_freq[i])
        out[2 * i] = vec[2 * i] * math.cos(a) - vec[2 * i + 1] * math.sin(a)
        out[2 * i + 1] = vec[2 * i] * math.sin(a) + vec[2 * i + 1] * math.cos(a)
    return out


def _rms_loops(v, g, eps):
    ms = sum(e * e for e in v) / len(v)
    return [v[i] / math.sqrt(ms + eps) * g[i] for i in range(len(v))]


def _layer_loops(W, x, d):
    """Scalar-loop MLA prefill written from the definitions, for tiny shapes only.  With
    d["act_quant"] each projection input row is rounded to bf16 and goes through the fp8
    quantiser first (both separately pinned)."""
    T, D = x.shape
    qz = (lambda v: list(O.quantize_mx_fp8(O.bf16_round(np.array([v], dtype=np.float64)))[2][0])) \
        if d.get("act_quant") else (lambda v: v)
    H, Lq, Lkv, dn, dr, dv = (d[k] for k in ("n_heads", "q_lora_rank", "kv_lora_rank", "qk_nope", "qk_rope", "v_dim"))
    dqk = dn + dr
    q = [[[0.0] * dqk for _ in range(H)] for _ in range(T)]
    K = [[[0.0] * dqk for _ in range(H)] for _ in range(T)]
    V = [[[0.0] * dv for _ in range(H)] for _ in range(T)]
    rows = []
    f = d.get("inv_freq")
    for t in range(T):
        xt = [x[t, i] for i in range(D)]
        if "input_norm_w" in W:
            xt = _rms_loops(xt, W["input_norm_w"], d["norm_eps"])
        xt = qz(xt)
        if Lq:
            cq = [sum(xt[i] * W["wq_a"][i, j] for i in range(D)) for j in range(Lq)]
            qin = qz(_rms_loops(cq, W["q_norm_w"], d["norm_eps"]))
        else:
            qin = xt
        qf = [sum(qin[j] * W["wq_b"][j, c] for j in range(len(qin))) for c in range(H * dqk)]
        for h in range(H):
            head = qf[h * dqk:(h + 1) * dqk]
            q[t][h] = head[:dn] + _rope_pair_loops(head[dn:], t, inv_freq=f)
        kva = [sum(xt[i] * W["wkv_a"][i, c] for i in range(D)) for c in range(Lkv + dr)]
        cn = _rms_loops(kva[:Lkv], W["kv_norm_w"], d["norm_eps"])
        p = _rope_pair_loops(kva[Lkv:], t, inv_freq=f)
        rows.append(cn + p)
        cq_ = qz(cn)
        for h in range(H):
            e = [sum(cq_[c] * W["wkv_b"][c, h * (dn + dv) + j] for c in range(Lkv)) for j in range(dn + dv)]
            K[t][h] = e[:dn] + p
            V[t][h] = e[dn:]
    o = [[[0.0] * dv for _ in range(H)] for _ in range(T)]
    for t in range(T):
        for h in range(H):
            s = [d["softmax_scale"] * sum(q[t][h][k] * K[j][h][k] for k in range(dqk)) for j in range(t + 1)]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            for k in range(dv):
                o[t][h][k] = sum(e[j] * V[j][h][k] for j in range(t + 1)) / z
    oq = [qz([o[t][h][k] for h in range(H) for k in range(dv)]) for t in range(T)]
    y = [[sum(oq[t][h * dv + k] * W["wo"][h * dv + k, n] for h in range(H) for k in range(dv)) for n in range(D)]
         for t in range(T)]
    return dict(q=np.array(q), k=np.array(K), v=np.array(V), rows=np.array(rows), o=np.array(o), y=np.array(y))


@pytest.mark.parametrize("Lq,extras,aq", [(5, False, False), (0, False, False), (5, True, False), (0, True, False),
                                          (5, True, True), (0, False, True)])
def test_prefill_matches_scalar_loops(Lq, extras, aq):
    """extras: the layer-input RMSNorm, a given two-pair frequency table in place of
    theta^(-2i/dr), and the score scale with YaRN's factor-4 magnitude."""
    W, d = _tiny_weights(11 + Lq, D=7, H=2, Lq=Lq, Lkv=6, dn=3, dr=4, dv=2, input_norm=extras)
    if extras:
        d["inv_freq"] = np.array([0.9, 0.004])
        d["softmax_scale"] = O.softmax_scale(3, 4, 4.0, 1.0)
    d["act_quant"] = aq
    x = synth.rng(12, "x").standard_normal((4, 7))
    ref = _layer_loops(W, x, d)
    got = O.mla_prefill(W, x, d)
    for k in ("q", "k", "v", "rows", "o", "y"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-11, atol=1e-12, err_msg=k)
    if aq:  # quantisation changes the result, within the E4M3 error scale
        plain = O.mla_prefill(W, x, dict(d, act_quant=False))
        rel = np.abs(plain["y"] - got["y"]).max() / np.abs(plain["y"]).max()
        assert 1e-4 < rel < 0.2, rel


def test_decode_equals_prefill_last_token():
    w = synth.WORKLOADS[1]
    W = O.decode_weights(synth.make_weights(w))
    d = O.dims_of(w.shape)
    x = O.decode_tensor("f32", synth.make_x(w, 9).data)
    pre = O.mla_prefill(W, x, d)
    for t in (0, 4, 8):
        dec = O.mla_decode(W, x[t:t + 1], [pre["rows"][:t]], d, head_chunk=3)
        for k in ("q", "rows", "o", "y"):
            np.testing.assert_allclose(dec[k][0], pre[k][t], rtol=1e-12, atol=1e-13, err_msg=f"{k} t={t}")


def test_absorbed_equals_expanded():
    """q_nope . k_nope = (q_nope W_UK) . c and sum p v = (sum p c) W_UV (atlas MlaWeights
    w_uk_t / w_uv fields; NKI decode QKV q_absorb_w parameter), so the absorbed decode
    must reproduce the expanded oracle to float64 rounding."""
    W, d = _tiny_weights(21, D=16, H=3, Lq=8, Lkv=10, dn=5, dr=4, dv=3)
    H, Lkv, dn, dv = 3, 10, 5, 3
    r = synth.rng(22, "abs")
    hist = [r.standard_normal((n, Lkv + 4)) for n in (1, 6, 13)]
    x = r.standard_normal((3, 16))
    ref = O.mla_decode(W, x, hist, d, head_chunk=2)
    q = ref["q"]
    wkv_b = W["wkv_b"].reshape(Lkv, H, dn + dv)
    for b in range(3):
        rows = np.concatenate([hist[b], ref["rows"][b:b + 1]])
        for h in range(H):
            W_UK = wkv_b[:, h, :dn].T          # [dn, Lkv]
            W_UV = wkv_b[:, h, dn:]            # [Lkv, dv]
            q_lat = q[b, h, :dn] @ W_UK
            s = d["softmax_scale"] * (rows[:, :Lkv] @ q_lat + rows[:, Lkv:] @ q[b, h, dn:])
            p = np.exp(s - s.max())
            p /= p.sum()
            o = (p @ rows[:, :Lkv]) @ W_UV
            np.testing.assert_allclose(o, ref["o"][b, h], rtol=1e-12, atol=1e-14)


def test_fp8_weights_decode_exactly():
    """2^k block scales make dequantisation exact: the decoded weight times 2^-k is an E4M3FN value."""
    w = synth.WORKLOADS[5]
    t = synth.encode(synth.rng(5, "probe").standard_normal((300, 260)).astype(np.float32) * 0.02, "fp8", 5, "probe")
    dec = O.decode_tensor("fp8", t.data, t.scale)
    full = np.repeat(np.repeat(t.scale, 128, 0), 128, 1)[:300, :260].astype(np.float64)
    grid = np.array([O.e4m3fn_value(c) for c in range(256)])
    assert np.isin(dec / full, grid).all()
    assert set(np.log2(t.scale).ravel().astype(int)) <= {-4, -3, -2, -1, 0}


@pytest.mark.parametrize("P", [0, 5, 9])
def test_chunk_attention_equals_whole_prefill(P):
    """Attention of tokens P..N-1 over the prefix 0..P-1 equals the same tokens' output of one
    prefill of all N tokens (scalar loops pin that prefill); a one-token chunk equals decode."""
    W, d = _tiny_weights(31, D=7, H=2, Lq=5, Lkv=6, dn=3, dr=4, dv=2, input_norm=True)
    x = synth.rng(32, "x").standard_normal((12, 7))
    ref = _layer_loops(W, x, d)
    got = O.chunk_attention(W, ref["q"][P:], ref["rows"][:P], ref["rows"][P:], d, head_chunk=1)
    np.testing.assert_allclose(got, ref["o"][P:], rtol=1e-11, atol=1e-12)
    one = O.chunk_attention(W, ref["q"][11:12], ref["rows"][:11], ref["rows"][11:12], d)
    dec = O.decode_attention(W, ref["q"][11:12], [ref["rows"][:12]], d)
    np.testing.assert_allclose(one, dec, rtol=1e-13, atol=1e-14)
