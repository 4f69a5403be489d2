"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a fact the pages or the mathematics fix:
hand-worked values (tests/golden), closed forms, textbook special cases, a
library routine (torch's CPU float8/bfloat16 decoding) or pure-Python brute force
on tiny shapes.  Inputs come from ``synth``; nothing here touches the HIP library.
"""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------- storage formats
def test_e4m3fn_golden_points():
    for code_hex, val in _golden_rows("e4m3fn_points.txt"):
        got = O.e4m3fn_value(int(code_hex, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code_hex


def test_e4m3fn_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3fn_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()


def test_fp8_block_scale_indexing():
    """Every code 0x38 (= 1.0): the decoded weight is the scale of the 128x128 block."""
    K, N = 200, 300
    scale = np.array([[1, 2, 4], [8, 16, 32]], np.float32)
    d = O.decode_tensor("fp8", np.full((K, N), 0x38, np.uint8), scale)
    assert d[0, 0] == 1 and d[127, 127] == 1 and d[127, 128] == 2 and d[0, 299] == 4
    assert d[128, 0] == 8 and d[199, 255] == 16 and d[199, 256] == 32


def test_bf16_decode_matches_torch_and_synth_rounding():
    x = synth.rng(99, "bf16").standard_normal(4096).astype(np.float32) * 37
    bits = synth.bf16_bits(x)
    ref_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bits == ref_bits).all()
    ref_vals = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert (O.decode_tensor("bf16", bits) == ref_vals).all()


def test_synth_fp8_encoding_matches_torch_cast():
    v = synth.rng(98, "fp8").standard_normal(20000) * 60
    codes = synth.e4m3fn_encode(v)
    ref = torch.from_numpy(v.astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    assert (codes == ref.view(torch.uint8).numpy()).all()


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    eps = 1e-6
    # constant vector c: output c / sqrt(c^2 + eps) * gamma
    x = np.full((1, 7), 3.0)
    g = np.linspace(0.5, 1.5, 7)
    np.testing.assert_allclose(O.rms_norm(x, g, eps), (3.0 / math.sqrt(9.0 + eps) * g)[None], rtol=1e-14)
    # [3, 4]: mean square 12.5
    np.testing.assert_allclose(O.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), eps),
                               [[3 / math.sqrt(12.5 + eps), 4 / math.sqrt(12.5 + eps)]], rtol=1e-14)
    # gamma = 1: mean square of the output is ms / (ms + eps)
    z = synth.rng(1, "rms").standard_normal((5, 64)) * 1e-3
    ms = np.mean(z * z, axis=-1)
    out = O.rms_norm(z, np.ones(64), eps)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), ms / (ms + eps), rtol=1e-12)
    # scale invariance for large inputs (eps negligible)
    np.testing.assert_allclose(O.rms_norm(z * 1e6, g[0], eps), O.rms_norm(z * 2e6, g[0], eps), rtol=1e-9)


# ----------------------------------------------------------------------------- fp8 activation quantisation
def test_e4m3fn_round_matches_torch_cast():
    """Round-to-nearest-even into E4M3FN against torch's CPU float8 cast, on float32 values:
    every representable value, every midpoint between neighbours (the ties), and random
    values over the normal and subnormal ranges."""
    mags = np.array([O.e4m3fn_value(c) for c in range(0x7F)])
    mids = (mags[1:] + mags[:-1]) / 2
    r = synth.rng(5, "e4m3-round")
    rnd = np.concatenate([r.uniform(-448, 448, 4000), r.uniform(-2.0 ** -5, 2.0 ** -5, 2000),
                          r.uniform(-1, 1, 2000)])
    v = np.concatenate([mags, -mags, mids, -mids, rnd]).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3fn_round(v)
    assert (got == want).all(), np.nonzero(got != want)[0][:10]


def test_bf16_round_matches_torch_cast():
    """Round to nearest even into bfloat16 against torch's CPU cast of float32 values (every
    float32 is exact in float64, and bf16 rounding of a float32 is a single rounding)."""
    r = synth.rng(8, "bf16-round")
    v = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                        (1 + (2 * np.arange(1, 200) + 1) * 2.0 ** -9),      # exact ties
                        -(1 + (2 * np.arange(1, 200) + 1) * 2.0 ** -9), [0.0, -0.0]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(v.astype(np.float64))
    assert np.array_equal(got, want)


def test_quantize_mx_fp8_closed_forms():
    K = 300  # two full groups and a partial one of 44 columns
    x = np.zeros((5, K))
    x[0, :128] = np.linspace(-448.0, 448.0, 128) * 2.0 ** 3      # amax = 448 * 2^3 exactly -> e = 3
    x[0, 128:256] = 448.0 * 2.0 ** -7 * (1 + 2.0 ** -20)          # just above 448 * 2^-7 -> e = -6
    x[1, :128] = 1.0                                              # amax 1 -> e = -8 (448 * 2^-9 < 1 <= 448 * 2^-8)
    x[2, 256:] = 3.0                                              # partial group
    codes, exps, deq = O.quantize_mx_fp8(x)
    assert exps.shape == (5, 3)
    assert exps[0, 0] == 3 and exps[0, 1] == -6 and exps[1, 0] == -8 and exps[2, 2] == -7
    assert (exps[3] == 0).all() and (codes[3] == 0).all() and (deq[3] == 0).all()   # all-zero groups
    # values already of the form code * 2^e come back exactly
    table = np.array([O.e4m3fn_value(c) for c in range(256)])
    r = synth.rng(6, "mx")
    cs = r.integers(0, 256, (4, 256))
    cs[(cs & 0x7F) == 0x7F] = 0x38                                 # no NaN codes
    cs[:, 0] = 0x7E                                                # each group holds the largest code
    cs[:, 128] = 0xFE
    e_true = r.integers(-12, 6, (4, 2))
    xv = table[cs] * 2.0 ** np.repeat(e_true, 128, axis=1)
    c2, e2, d2 = O.quantize_mx_fp8(xv)
    assert (e2 == e_true).all() and (d2 == xv).all()
    # error bound: half a unit of E4M3's 3-bit mantissa, or of the subnormal step 2^(e-9)
    z = r.standard_normal((6, 384)) * np.array([1e-3, 1.0, 50.0, 1e4, 1e-8, 3.0])[:, None]
    c3, e3, d3 = O.quantize_mx_fp8(z)
    sc = 2.0 ** np.repeat(e3, 128, axis=1)
    assert (np.abs(d3 - z) <= np.maximum(np.abs(z) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-12)).all()
    assert (np.abs(z / sc) <= 448).all()


# ----------------------------------------------------------------------------- RoPE
def test_rope_golden_points():
    for row in _golden_rows("rope_points.txt"):
        vals = [float(v) for v in row]
        pos, x, y = vals[0], np.array(vals[1:5]), np.array(vals[5:9])
        got = O.rope_interleaved(x[None], O.rope_angles(np.array([pos]), 4))[0]
        np.testing.assert_allclose(got, y, atol=1e-15)


def test_rope_pairing_is_interleaved_not_half_split():
    dr = 8
    x = np.zeros((1, dr))
    x[0, 1] = 1.0
    y = O.rope_interleaved(x, O.rope_angles(np.array([3]), dr))[0]
    assert set(np.nonzero(np.abs(y) > 1e-12)[0]) <= {0, 1}
    x = np.zeros((1, dr))
    x[0, 2] = 1.0  # pair 1 -> indices {2, 3}; a half-split rope would use {2, 6}
    y = O.rope_interleaved(x, O.rope_angles(np.array([3]), dr))[0]
    assert set(np.nonzero(np.abs(y) > 1e-12)[0]) == {2, 3}


def test_rope_invariants():
    dr = 64
    r = synth.rng(2, "rope")
    q, k = r.standard_normal(dr), r.standard_normal(dr)
    pos = np.array([0, 5, 17, 1000, 32767])
    ang = O.rope_angles(pos, dr)
    Q = O.rope_interleaved(np.tile(q, (len(pos), 1)), ang)
    K = O.rope_interleaved(np.tile(k, (len(pos), 1)), ang)
    np.testing.assert_allclose(Q[0], q, atol=0)                       # position 0 is the identity
    np.testing.assert_allclose(np.linalg.norm(Q.reshape(len(pos), -1, 2), axis=-1),
                               np.linalg.norm(q.reshape(-1, 2), axis=-1)[None].repeat(len(pos), 0), rtol=1e-12)
    # <R_m q, R_n k> depends only on m - n
    a = O.rope_interleaved(np.stack([q, q]), O.rope_angles(np.array([22, 1005]), dr))
    b = O.rope_interleaved(np.stack([k, k]), O.rope_angles(np.array([17, 1000]), dr))
    assert abs(a[0] @ b[0] - a[1] @ b[1]) < 1e-9
    # multi-head broadcast: every head rotated by its token's angle
    qh = r.standard_normal((3, 4, dr))
    out = O.rope_interleaved(qh, O.rope_angles(np.array([1, 2, 3]), dr))
    for t in range(3):
        for h in range(4):
            np.testing.assert_allclose(out[t, h], O.rope_interleaved(qh[t:t + 1, h], O.rope_angles(np.array([t + 1]), dr))[0])


# ----------------------------------------------------------------------------- YaRN
def _turns(rope_dim, theta, L):
    """Full turns pair i makes over L positions when it advances theta^(-2i/d) rad per position."""
    return np.array([L * theta ** (-2.0 * i / rope_dim) / (2 * math.pi) for i in range(rope_dim // 2)])


def test_yarn_factor_one_is_plain_rope():
    for dr in (16, 64):
        np.testing.assert_allclose(O.yarn_inv_freq(dr, 10000.0, 1.0, 4096),
                                   [10000.0 ** (-2 * i / dr) for i in range(dr // 2)], rtol=1e-15)
    assert O.yarn_mscale(1.0, 1.0) == 1.0 and O.yarn_mscale(0.5, 3.0) == 1.0
    assert O.softmax_scale(128, 64, 1.0, 1.0) == O.softmax_scale(128, 64)


@pytest.mark.parametrize("dr,theta,s,L,bf,bs", [(64, 1e4, 40.0, 4096, 32.0, 1.0), (64, 1e4, 4.0, 2048, 32.0, 1.0),
                                                (128, 5e5, 8.0, 8192, 16.0, 2.0), (16, 1e4, 8.0, 256, 32.0, 1.0)])
def test_yarn_regions_follow_turn_counts(dr, theta, s, L, bf, bs):
    """Kept iff the pair turns >= beta_fast times over the original context, divided by the
    factor iff it turns <= beta_slow times, blended in between with the interpolated share
    growing in equal steps from the last kept pair to the first interpolated one."""
    plain = np.array([theta ** (-2.0 * i / dr) for i in range(dr // 2)])
    turns = _turns(dr, theta, L)
    f = O.yarn_inv_freq(dr, theta, s, L, bf, bs)
    keep, interp = turns >= bf, turns <= bs
    assert keep.any() and interp.any()
    np.testing.assert_allclose(f[keep], plain[keep], rtol=1e-15)
    np.testing.assert_allclose(f[interp], plain[interp] / s, rtol=1e-15)
    mid = ~keep & ~interp
    share = (plain[mid] - f[mid]) / (plain[mid] - plain[mid] / s)
    assert ((share > 0) & (share < 1)).all()
    steps = np.diff(np.concatenate([[0.0], share, [1.0]]))
    np.testing.assert_allclose(steps, 1.0 / (mid.sum() + 1), rtol=1e-9)


def test_yarn_v3_golden():
    g = {k: float(v) for k, v in _golden_rows("yarn_v3.txt")}
    plain = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    f = O.yarn_inv_freq(64, 10000.0, 40.0, 4096, 32.0, 1.0)
    kept = np.nonzero(np.isclose(f, plain, rtol=1e-15, atol=0))[0]
    interp = np.nonzero(np.isclose(f, plain / 40.0, rtol=1e-15, atol=0))[0]
    assert kept.max() == g["last_kept_pair"] and (kept == np.arange(kept.max() + 1)).all()
    assert interp.min() == g["first_interpolated_pair"] and (interp == np.arange(interp.min(), 32)).all()
    assert O.yarn_mscale(40.0, 1.0) == pytest.approx(g["mscale"], rel=1e-15)
    assert O.softmax_scale(128, 64, 40.0, 1.0) == pytest.approx(g["score_scale"], rel=1e-15)
    assert O.yarn_mscale(math.exp(10.0), 1.0) == pytest.approx(2.0, rel=1e-15)
    assert O.yarn_mscale(math.exp(10.0), 0.5) == pytest.approx(1.5, rel=1e-15)
    d = O.dims_of(synth.custom(synth.WORKLOADS[3], 120, "yarn", rope_factor=40.0).shape)
    np.testing.assert_array_equal(d["inv_freq"], f)
    assert d["softmax_scale"] == pytest.approx(g["score_scale"], rel=1e-15)


def test_rope_with_yarn_table_invariants():
    dr = 64
    f = O.yarn_inv_freq(dr, 10000.0, 40.0, 4096)
    r = synth.rng(4, "rope-yarn")
    q, k = r.standard_normal(dr), r.standard_normal(dr)
    ang = O.rope_angles(np.array([0, 7, 40000]), dr, inv_freq=f)
    np.testing.assert_allclose(ang[1], 7 * f, rtol=1e-15)
    Q = O.rope_interleaved(np.tile(q, (3, 1)), ang)
    np.testing.assert_allclose(Q[0], q, atol=0)
    a = O.rope_interleaved(np.stack([q, q]), O.rope_angles(np.array([22, 30005]), dr, inv_freq=f))
    b = O.rope_interleaved(np.stack([k, k]), O.rope_angles(np.array([17, 30000]), dr, inv_freq=f))
    assert abs(a[0] @ b[0] - a[1] @ b[1]) < 1e-9


# ----------------------------------------------------------------------------- layer-input RMSNorm
def test_input_norm_closed_form():
    """Rows that are constant vectors c*1 normalise to c/sqrt(c^2+eps)*gamma, so a layer with
    input_norm_w equals the layer without it fed with that closed form."""
    w = synth.custom(synth.WORKLOADS[1], 121, "input-norm", input_norm=True)
    W = O.decode_weights(synth.make_weights(w))
    d = O.dims_of(w.shape)
    cs = np.array([0.5, -3.0, 1e-2, 7.25])
    x = cs[:, None] * np.ones((1, w.shape.hidden))
    xn = (cs / np.sqrt(cs * cs + 1e-6))[:, None] * W["input_norm_w"][None]
    plain = {k: v for k, v in W.items() if k != "input_norm_w"}
    pos = np.array([0, 3, 9, 200])
    q1, r1 = O.project(W, x, pos, d)
    q2, r2 = O.project(plain, xn, pos, d)
    np.testing.assert_allclose(q1, q2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r1, r2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(O.project_rows(W, x, pos, d), r2, rtol=1e-12, atol=1e-14)
    # without the gamma the layer differs (the fold is not a no-op)
    assert np.abs(O.project(plain, x, pos, d)[0] - q1).max() > 1e-3


# ----------------------------------------------------------------------------- softmax attention
def _attention_loops(q, K, V, scale, qpos):
    Tq, H, _ = q.shape
    out = np.zeros((Tq, H, V.shape[2]))
    for i in range(Tq):
        for h in range(H):
            js = [j for j in range(K.shape[0]) if j <= qpos[i]]
            s = [scale * sum(q[i, h, d] * K[j, h, d] for d in range(q.shape[2])) for j in js]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            for d in range(V.shape[2]):
                out[i, h, d] = sum(e[n] * V[js[n], h, d] for n in range(len(js))) / z
    return out


def test_attention_brute_force_and_special_cases():
    r = synth.rng(3, "attn")
    q, K, V = r.standard_normal((5, 3, 6)), r.standard_normal((5, 3, 6)), r.standard_normal((5, 3, 4))
    pos = np.arange(5)
    got = O.attention(q, K, V, 0.4, pos)
    np.testing.assert_allclose(got, _attention_loops(q, K, V, 0.4, pos), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got[0], V[0], rtol=1e-15)               # causal query 0 sees only key 0
    Ke = np.repeat(K[:1], 5, axis=0)                                     # all keys equal: mean of V
    np.testing.assert_allclose(O.attention(q, Ke, V, 0.4, np.array([4] * 5)),
                               np.repeat(V.mean(0, keepdims=True), 5, 0), rtol=1e-12)
    np.testing.assert_allclose(O.attention(q, K, np.ones((5, 3, 4)), 0.4, pos), 1.0, rtol=1e-14)


def test_scale_and_example_dims_golden():
    g = {k: float(v) for k, v in _golden_rows("dims.txt")}
    assert g["qk_head"] == g["qk_nope"] + g["qk_rope"]
    assert O.softmax_scale(32, 16) == pytest.approx(g["scale_qk48"], rel=1e-15)
    assert O.softmax_scale(128, 64) == pytest.approx(g["scale_qk192"], rel=1e-15)
    s = synth.WORKLOADS[3].shape
    assert (s.q_lora_rank, s.kv_lora_rank, s.qk_nope, s.qk_rope, s.v_dim) == \
        (g["q_lora_rank"], g["kv_lora_rank"], g["qk_nope"], g["qk_rope"], g["v_dim"])


# ----------------------------------------------------------------------------- paging
def test_paging_bijection_integer_only():
    w = synth.WORKLOADS[3]
    ctx = np.array([1, 63, 64, 65, 200, 7])
    p = synth.make_paging(7, ctx, 64, spare=5)
    used = p.block_table[p.block_table >= 0]
    assert len(np.unique(used)) == len(used) and used.max() < p.n_blocks
    # each token's row encodes its (sequence, position); placement must be a bijection
    cache = np.full((p.n_blocks, 64, 2), -1, np.int64)
    for b, n in enumerate(ctx):
        rows = np.stack([np.full(n, b), np.arange(n)], axis=1)
        slots = synth.slots_for(p.block_table[b], np.arange(n), 64)
        cache = O.place_rows(cache, slots, rows)
    assert (cache[..., 0] >= 0).sum() == ctx.sum()
    for b, n in enumerate(ctx):
        dense = O.cache_read_dense(cache, p.block_table[b], n, 64)
        assert (dense[:, 0] == b).all() and (dense[:, 1] == np.arange(n)).all()
    # synth.fill_cache agrees with the oracle's placement model
    c2 = np.full_like(cache, -1)
    for b, n in enumerate(ctx):
        synth.fill_cache(c2, p, b, np.stack([np.full(n, b), np.arange(n)], axis=1))
    assert (c2 == cache).all()
    # decode slot of sequence b is the row of position ctx-1; slot -1 skips
    sm = synth.decode_slot_mapping(p)
    for b, n in enumerate(ctx):
        assert tuple(cache.reshape(-1, 2)[sm[b]]) == (b, n - 1)
    same = O.place_rows(cache, np.array([-1]), np.array([[9, 9]]))
    assert (same == cache).all()
