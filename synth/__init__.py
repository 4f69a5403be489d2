"""Seeded synthetic inputs for the MLA hot path.

This module is shared by the CPU oracle (``oracle/``) and the HIP path (the
``head_latent_attention_amd`` binding, ``bench.py``).  It holds no arithmetic of
the attention method itself: it only draws random numbers, encodes them in the
storage formats the library consumes (fp32, bf16 bit patterns, OCP E4M3FN codes
with power-of-two block scales) and lays out paging metadata (block tables,
slot mappings, context lengths).  Every array is a pure function of
(config number, tensor name), so generation order never changes a value.

Distributions follow the workloads the pages describe:
  * weights ~ N(0, 0.02)  (NeMo ``MLA.init_weights`` default ``init_std``),
  * RMSNorm gammas ~ 1 + N(0, 0.1),
  * hidden states x ~ N(0, 1),
  * fp8 weights: codes = E4M3FN(W / 2^k), one k ~ U{-4..0} per 128x128 block,
    the block-scaled FP8-E4M3 format of the atlas ``MlaWeights`` fp8 fields.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import numpy as np

F32, BF16, FP8 = "f32", "bf16", "fp8"


@dataclasses.dataclass(frozen=True)
class MlaShape:
    """Dimensions of one MLA layer, named as in the logicaffeine ``Mla`` struct."""
    hidden: int
    n_heads: int
    q_lora_rank: int          # 0 = full query projection (no q latent)
    kv_lora_rank: int
    qk_nope: int
    qk_rope: int
    v_dim: int
    act: str                  # F32 | BF16  (x, q, k, v, o, y, cache rows)
    weight: str               # F32 | BF16 | FP8
    block_size: int = 64
    rope_theta: float = 10000.0
    norm_eps: float = 1e-6
    # YaRN context extension (factor 1 = plain RoPE); the values of the other fields are
    # the published DeepSeek-V3 rope-scaling settings
    rope_factor: float = 1.0
    rope_original_max: int = 4096
    rope_beta_fast: float = 32.0
    rope_beta_slow: float = 1.0
    rope_mscale_all_dim: float = 1.0
    input_norm: bool = False  # the layer-input RMSNorm gamma input_norm_w is given
    act_quant: bool = False   # activations entering the projections are fp8-quantised

    @property
    def qk_head(self) -> int:
        return self.qk_nope + self.qk_rope

    @property
    def row(self) -> int:
        return self.kv_lora_rank + self.qk_rope


@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    shape: MlaShape
    kind: str                 # "prefill+decode" | "prefill" | "decode"
    T: int = 0                # prefill tokens
    decode_steps: int = 0     # C1: decode steps after the prefill
    B: int = 0                # decode batch
    ctx_dist: str = ""        # "uniform" | "loguniform"
    ctx_lo: int = 0
    ctx_hi: int = 0


V3 = dict(hidden=7168, n_heads=128, q_lora_rank=1536, kv_lora_rank=512,
          qk_nope=128, qk_rope=64, v_dim=128)

WORKLOADS = {
    1: Workload(1, "tiny-fp32", MlaShape(256, 4, 64, 64, 32, 16, 32, F32, F32, block_size=16),
                "prefill+decode", T=64, decode_steps=16, B=1),
    2: Workload(2, "v2lite-prefill-4096", MlaShape(2048, 16, 0, 512, 128, 64, 128, BF16, BF16),
                "prefill", T=4096),
    3: Workload(3, "v3-decode-b64", MlaShape(**V3, act=BF16, weight=BF16), "decode", B=64,
                ctx_dist="uniform", ctx_lo=1024, ctx_hi=8192),
    4: Workload(4, "v3-prefill-8192", MlaShape(**V3, act=BF16, weight=BF16), "prefill", T=8192),
    5: Workload(5, "v3-decode-fp8-b256", MlaShape(**V3, act=BF16, weight=FP8), "decode", B=256,
                ctx_dist="loguniform", ctx_lo=512, ctx_hi=32768),
}


def rng(cfg_no: int, name: str) -> np.random.Generator:
    """One independent stream per (config, tensor name)."""
    return np.random.default_rng(np.random.SeedSequence([cfg_no, zlib.crc32(name.encode())]))


# ----------------------------------------------------------------------------- encodings
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3fn_grid() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, indexed by code 0..126 (increasing)."""
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e - 7.0))


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Round float values to OCP E4M3FN codes: nearest, ties to even code, saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    grid = _e4m3fn_grid()
    a = np.minimum(np.abs(v), grid[-1])
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == grid[hi], hi, code).astype(np.uint8)
    return np.where(v < 0, code | 0x80, code).astype(np.uint8)


@dataclasses.dataclass
class Tensor:
    """A host array in the library's storage format.

    kind F32: ``data`` float32.  BF16: ``data`` uint16 bit patterns.
    FP8: ``data`` uint8 E4M3FN codes, ``scale`` float32 [ceil(K/128), ceil(N/128)].
    """
    kind: str
    data: np.ndarray
    scale: Optional[np.ndarray] = None


def encode(x: np.ndarray, kind: str, cfg_no: int = 0, name: str = "") -> Tensor:
    if kind == F32:
        return Tensor(F32, np.ascontiguousarray(x, dtype=np.float32))
    if kind == BF16:
        return Tensor(BF16, bf16_bits(x))
    if kind == FP8:
        K, N = x.shape
        kb, nb = -(-K // 128), -(-N // 128)
        k = rng(cfg_no, name + ".scale_exp").integers(-4, 1, size=(kb, nb))
        scale = np.ldexp(np.ones((kb, nb), np.float32), k).astype(np.float32)
        full = np.repeat(np.repeat(scale, 128, 0), 128, 1)[:K, :N]
        return Tensor(FP8, e4m3fn_encode(x / full), scale)
    raise ValueError(kind)


# ----------------------------------------------------------------------------- weights
WEIGHT_NAMES = ("wq_a", "wq_b", "wkv_a", "wkv_b", "wo")


def weight_shapes(s: MlaShape) -> dict:
    qin = s.q_lora_rank if s.q_lora_rank else s.hidden
    shapes = {
        "wq_b": (qin, s.n_heads * s.qk_head),
        "wkv_a": (s.hidden, s.row),
        "wkv_b": (s.kv_lora_rank, s.n_heads * (s.qk_nope + s.v_dim)),
        "wo": (s.n_heads * s.v_dim, s.hidden),
    }
    if s.q_lora_rank:
        shapes["wq_a"] = (s.hidden, s.q_lora_rank)
    return shapes


def make_weights(w: Workload) -> dict:
    """Weights in [in, out] row-major orientation plus fp32 gammas.

    Returns {name: Tensor}; gammas are float32 arrays (already bf16-representable
    when the activations are bf16)."""
    s = w.shape
    out = {}
    for name, shp in weight_shapes(s).items():
        g = rng(w.number, name).standard_normal(shp, dtype=np.float32) * np.float32(0.02)
        out[name] = encode(g, s.weight, w.number, name)
    gammas = [("q_norm_w", s.q_lora_rank), ("kv_norm_w", s.kv_lora_rank)]
    if s.input_norm:
        gammas.append(("input_norm_w", s.hidden))
    for name, n in gammas:
        if n == 0:
            continue
        g = (1.0 + 0.1 * rng(w.number, name).standard_normal(n)).astype(np.float32)
        if s.act == BF16:
            g = bf16_bits_to_f32(bf16_bits(g))
        out[name] = Tensor(F32, g)
    return out


def make_x(w: Workload, rows: int, name: str = "x") -> Tensor:
    x = rng(w.number, name).standard_normal((rows, w.shape.hidden), dtype=np.float32)
    return encode(x, w.shape.act)


# ----------------------------------------------------------------------------- paging
def shuffled_blocks(cfg_no: int, name: str, n_blocks: int) -> np.ndarray:
    return rng(cfg_no, name).permutation(n_blocks).astype(np.int32)


def slots_for(block_table_row: np.ndarray, positions: np.ndarray, bs: int) -> np.ndarray:
    """Flat cache row of each position of one sequence: block_table[pos // bs] * bs + pos % bs."""
    positions = np.asarray(positions, dtype=np.int64)
    return (block_table_row[positions // bs].astype(np.int64) * bs + positions % bs).astype(np.int32)


def context_lengths(w: Workload) -> np.ndarray:
    r = rng(w.number, "context_lens")
    if w.ctx_dist == "uniform":
        return r.integers(w.ctx_lo, w.ctx_hi + 1, size=w.B).astype(np.int32)
    if w.ctx_dist == "loguniform":
        u = r.uniform(np.log(w.ctx_lo), np.log(w.ctx_hi), size=w.B)
        return np.clip(np.rint(np.exp(u)), w.ctx_lo, w.ctx_hi).astype(np.int32)
    raise ValueError(w.ctx_dist)


@dataclasses.dataclass
class Paging:
    block_table: np.ndarray    # int32 [B, max_blocks], -1 padded
    context_lens: np.ndarray   # int32 [B]
    n_blocks: int              # physical blocks in the cache
    block_size: int


def make_paging(cfg_no: int, ctx: np.ndarray, bs: int, spare: int = 64, name: str = "blocks") -> Paging:
    """A random permutation of physical blocks shared out over sequences, tables -1 padded."""
    ctx = np.asarray(ctx, dtype=np.int64)
    need = -(-ctx // bs)
    total = int(need.sum())
    n_blocks = total + spare
    perm = shuffled_blocks(cfg_no, name, n_blocks)
    max_blocks = int(need.max())
    table = np.full((len(ctx), max_blocks), -1, np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return Paging(table, ctx.astype(np.int32), n_blocks, bs)


def decode_slot_mapping(p: Paging) -> np.ndarray:
    """The new token of sequence b sits at position context_lens[b] - 1."""
    pos = p.context_lens.astype(np.int64) - 1
    return np.array([slots_for(p.block_table[b], pos[b:b + 1], p.block_size)[0]
                     for b in range(len(pos))], np.int32)


def history_rows(w: Workload, b: int, n: int) -> Tensor:
    """Dense latent-cache history [n, R] of sequence b: c ~ N(0,1), k_pe ~ N(0, 1.7^2).

    These are the magnitudes the projection front end gives at V3 shapes (a
    normalised latent with gamma ~ 1, and a rope key of std 0.02*sqrt(hidden))."""
    s = w.shape
    r = rng(w.number, f"history.{b}")
    rows = r.standard_normal((n, s.row), dtype=np.float32)
    rows[:, s.kv_lora_rank:] *= np.float32(0.02 * np.sqrt(s.hidden))
    return encode(rows, s.act)


def fill_cache(cache: np.ndarray, p: Paging, b: int, rows: np.ndarray) -> None:
    """Write sequence b's dense rows [n, R] into cache [n_blocks, bs, R] through its table."""
    n = rows.shape[0]
    slots = slots_for(p.block_table[b], np.arange(n), p.block_size).astype(np.int64)
    flat = cache.reshape(-1, cache.shape[-1])
    flat[slots] = rows


# ----------------------------------------------------------------------------- per-entry-point inputs
def make_normal(w: Workload, name: str, shape, std: float = 1.0) -> Tensor:
    """N(0, std^2) activations of the given shape in the workload's activation format
    (used for the q/k/v/o inputs of the attention and output-projection entry points)."""
    x = rng(w.number, name).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return encode(x, w.shape.act)


def custom(base: Workload, number: int, name: str, **changes) -> Workload:
    """A variant workload (edge-case sizes) with its own seed number."""
    shape_keys = {f.name for f in dataclasses.fields(MlaShape)}
    sh = dataclasses.replace(base.shape, **{k: v for k, v in changes.items() if k in shape_keys})
    rest = {k: v for k, v in changes.items() if k not in shape_keys}
    return dataclasses.replace(base, number=number, name=name, shape=sh, **rest)
