"""ctypes binding of libmla.so: argument marshalling only.

Each function has the name of the C entry point it calls, takes torch tensors
that already live on the GPU, passes their raw pointers and the current HIP
stream, and raises :class:`MlaError` on a non-zero status.  All computation
happens in the library's HIP kernels; torch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Dict, Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
FN_QKV_PREFILL, FN_PREFILL_ATTN, FN_DECODE_QKV, FN_DECODE_ATTN, FN_OUT_PROJ, FN_PREFILL_ATTN_PAGED = range(6)
_DTYPES = {"f32": MLA_F32, "bf16": MLA_BF16, "fp8": MLA_FP8_E4M3}
SYMBOLS = ("mla_qkv_prefill", "mla_prefill_attn", "mla_decode_qkv_and_scatter", "mla_decode_attn_absorbed",
           "mla_out_proj", "mla_prefill_attn_paged", "mla_quantize_fp8", "mla_rope_inv_freq", "mla_rope_tables",
           "mla_decode_attn_absorbed_noalloc", "mla_workspace_size", "mla_status_string", "mla_rope_score_scale")
_STATUS_FNS = SYMBOLS[:10]
NOALLOC_SCRATCH_BYTES = 64 << 20   # MLA_NOALLOC_SCRATCH_MIB of include/mla.h


class MlaError(RuntimeError):
    pass


class MlaConfig(Structure):
    _fields_ = [("hidden", c_int32), ("n_heads", c_int32), ("q_lora_rank", c_int32), ("kv_lora_rank", c_int32),
                ("qk_nope", c_int32), ("qk_rope", c_int32), ("v_dim", c_int32), ("softmax_scale", c_float),
                ("norm_eps", c_float), ("block_size", c_int32), ("act_dtype", c_int32), ("weight_dtype", c_int32),
                ("act_quant", c_int32)]


class MlaWeight(Structure):
    _fields_ = [("w", c_void_p), ("scale", c_void_p)]


class MlaWeights(Structure):
    _fields_ = [("wq_a", MlaWeight), ("wq_b", MlaWeight), ("wkv_a", MlaWeight), ("wkv_b", MlaWeight),
                ("wo", MlaWeight), ("q_norm_w", c_void_p), ("kv_norm_w", c_void_p), ("input_norm_w", c_void_p)]


class MlaRope(Structure):
    _fields_ = [("theta", c_double), ("factor", c_double), ("original_max_position", c_int32),
                ("beta_fast", c_double), ("beta_slow", c_double), ("mscale_all_dim", c_double)]


def rope(theta=10000.0, factor=1.0, original_max_position=4096, beta_fast=32.0, beta_slow=1.0,
         mscale_all_dim=1.0) -> MlaRope:
    """Rotary settings: plain RoPE with base theta, or YaRN when factor > 1."""
    return MlaRope(theta, factor, original_max_position, beta_fast, beta_slow, mscale_all_dim)


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (built by head_latent_attention_amd.build); fails loudly if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m head_latent_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = c_void_p, c_int32, c_int64, c_size_t
    C, W = POINTER(MlaConfig), POINTER(MlaWeights)
    lib.mla_qkv_prefill.argtypes = [C, W, P, I32, P, P, P, P, P, P, P, I64, P, SZ, P]
    lib.mla_prefill_attn.argtypes = [C, P, P, P, I32, P, P, SZ, P]
    lib.mla_decode_qkv_and_scatter.argtypes = [C, W, P, I32, P, P, P, I64, P, P, P, SZ, P]
    lib.mla_decode_attn_absorbed.argtypes = [C, W, P, I32, P, I64, P, I32, P, P, P, SZ, P]
    lib.mla_out_proj.argtypes = [C, W, P, I32, P, P, SZ, P]
    lib.mla_prefill_attn_paged.argtypes = [C, W, P, I32, P, I64, P, I32, I32, P, P, SZ, P]
    lib.mla_decode_attn_absorbed_noalloc.argtypes = [C, W, P, I32, P, I64, P, I32, P, P, P]
    lib.mla_quantize_fp8.argtypes = [P, I32, I32, I64, P, P, P]
    lib.mla_rope_inv_freq.argtypes = [POINTER(MlaRope), I32, P, P]
    lib.mla_rope_tables.argtypes = [I32, I32, P, I32, P, P, P, P]
    lib.mla_rope_score_scale.argtypes = [POINTER(MlaRope), I32, I32]
    lib.mla_rope_score_scale.restype = c_double
    lib.mla_workspace_size.argtypes = [C, I32, I32, I32]
    lib.mla_workspace_size.restype = SZ
    lib.mla_status_string.argtypes = [I32]
    lib.mla_status_string.restype = c_char_p
    for name in _STATUS_FNS:
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def config(hidden, n_heads, q_lora_rank, kv_lora_rank, qk_nope, qk_rope, v_dim, *, act="bf16",
           weight="bf16", block_size=64, softmax_scale=None, norm_eps=1e-6, rope: Optional[MlaRope] = None,
           act_quant: bool = False) -> MlaConfig:
    """The layer's config; the score scale defaults to mla_rope_score_scale(rope) (1/sqrt(dqk)
    times YaRN's magnitude squared when rope has factor > 1)."""
    if softmax_scale is None:
        softmax_scale = load().mla_rope_score_scale(ctypes.byref(rope) if rope is not None else None,
                                                    qk_nope, qk_rope)
    return MlaConfig(hidden, n_heads, q_lora_rank or 0, kv_lora_rank, qk_nope, qk_rope, v_dim, softmax_scale,
                     norm_eps, block_size, _DTYPES[act], _DTYPES[weight], int(bool(act_quant)))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise MlaError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise MlaError("tensor must be contiguous")
    return t.data_ptr()


# ---- argument checks: the C ABI takes raw pointers, so dtypes and element counts are checked
# here, before the call (an int64 index tensor read as int32 pairs, or a buffer smaller than the
# shapes in include/mla.h, would otherwise go unnoticed)
_ACT_DTYPE = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}
_FP8_DTYPES = tuple(t for t in (torch.uint8, getattr(torch, "float8_e4m3fn", None)) if t is not None)


def _act_dtype(cfg: MlaConfig):
    return _ACT_DTYPE[cfg.act_dtype]


def _need(t, name: str, dtype, numel: Optional[int] = None, shape=None):
    """t must be a tensor of `dtype` (a dtype or a tuple of them) with `numel` elements, or of
    exactly `shape` (None entries match any size)."""
    if t is None:
        raise MlaError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise MlaError(f"{name} must be a torch tensor")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise MlaError(f"{name} must have dtype {' or '.join(str(d) for d in dts)}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(e is not None and e != a for e, a in zip(shape, t.shape)):
            raise MlaError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise MlaError(f"{name} must have {numel} elements, got {t.numel()}")


def _need_cache(cfg: MlaConfig, kv_cache):
    """The paged latent cache [n_blocks, 1, block_size, kv_lora_rank + qk_rope] in the act dtype."""
    _need(kv_cache, "kv_cache", _act_dtype(cfg),
          shape=(None, 1, cfg.block_size, cfg.kv_lora_rank + cfg.qk_rope))
    if kv_cache.shape[0] < 1:
        raise MlaError("kv_cache must hold at least one block")


def _need_tables(cfg: MlaConfig, cos, sin, n: int):
    for name, t in (("cos", cos), ("sin", sin)):
        _need(t, name, torch.float32, numel=n * (cfg.qk_rope // 2))


def _need_ws(ws):
    if ws is not None and not isinstance(ws, torch.Tensor):
        raise MlaError("ws must be a torch tensor")


def weight_shapes(cfg: MlaConfig) -> Dict[str, tuple]:
    """[in, out] shape of each projection weight and [n] of each fp32 gamma (include/mla.h)."""
    H, dqk = cfg.n_heads, cfg.qk_nope + cfg.qk_rope
    qin = cfg.q_lora_rank if cfg.q_lora_rank else cfg.hidden
    shp = {"wq_b": (qin, H * dqk), "wkv_a": (cfg.hidden, cfg.kv_lora_rank + cfg.qk_rope),
           "wkv_b": (cfg.kv_lora_rank, H * (cfg.qk_nope + cfg.v_dim)), "wo": (H * cfg.v_dim, cfg.hidden),
           "kv_norm_w": (cfg.kv_lora_rank,), "input_norm_w": (cfg.hidden,)}
    if cfg.q_lora_rank:
        shp["wq_a"] = (cfg.hidden, cfg.q_lora_rank)
        shp["q_norm_w"] = (cfg.q_lora_rank,)
    return shp


class Weights:
    """Holds the device tensors of one layer and their MlaWeights struct."""

    def __init__(self, tensors: Dict[str, torch.Tensor], scales: Optional[Dict[str, torch.Tensor]] = None):
        self.tensors = dict(tensors)
        self.scales = dict(scales or {})
        s = MlaWeights()
        for name in ("wq_a", "wq_b", "wkv_a", "wkv_b", "wo"):
            t = self.tensors.get(name)
            sc = self.scales.get(name)
            setattr(s, name, MlaWeight(_ptr(t) if t is not None else None, _ptr(sc) if sc is not None else None))
        s.q_norm_w = _ptr(self.tensors.get("q_norm_w")) if "q_norm_w" in self.tensors else None
        s.kv_norm_w = _ptr(self.tensors.get("kv_norm_w"))
        s.input_norm_w = _ptr(self.tensors.get("input_norm_w"))
        self.struct = s

    def check(self, cfg: MlaConfig, names) -> None:
        """The weights an entry point reads match the config: dtype, shape, and for fp8 the fp32
        block-scale grid [ceil(K/128), ceil(N/128)]; gammas fp32.  Optional ones (input_norm_w)
        are checked only when present."""
        shapes = weight_shapes(cfg)
        wdt = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16, MLA_FP8_E4M3: _FP8_DTYPES}[cfg.weight_dtype]
        for name in names:
            if name not in shapes:
                continue
            t = self.tensors.get(name)
            if t is None and name == "input_norm_w":
                continue
            if name.endswith("_norm_w"):
                _need(t, name, torch.float32, numel=shapes[name][0])
                continue
            K, N = shapes[name]
            _need(t, name, wdt, shape=(K, N))
            if cfg.weight_dtype == MLA_FP8_E4M3:
                _need(self.scales.get(name), f"{name} scale", torch.float32, shape=(-(-K // 128), -(-N // 128)))


_FRONT = ("wq_a", "wq_b", "wkv_a", "q_norm_w", "kv_norm_w", "input_norm_w")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(st: int) -> None:
    if st != 0:
        raise MlaError(f"libmla status {st}: {load().mla_status_string(st).decode()}")


def workspace_size(cfg: MlaConfig, fn: int, n: int, max_context: int = 0) -> int:
    return int(load().mla_workspace_size(ctypes.byref(cfg), fn, n, max_context))


def workspace(cfg: MlaConfig, fn: int, n: int, max_context: int = 0, device="cuda") -> torch.Tensor:
    size = workspace_size(cfg, fn, n, max_context)
    return torch.empty(max(size, 1), dtype=torch.uint8, device=device)


def _ws(ws, cfg, fn, n, max_context=0, device="cuda"):
    _need_ws(ws)
    if ws is None:
        ws = workspace(cfg, fn, n, max_context, device)
    return ws, ws.numel() * ws.element_size()


def mla_quantize_fp8(x, stream=None):
    """MX fp8 codes [M, K] (uint8) and exponent bytes [ceil(K/128), M] (e + 127) of bf16 rows x."""
    _need(x, "x", torch.bfloat16, shape=(None, None))
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    exps = torch.empty(((K + 127) // 128, M), dtype=torch.uint8, device=x.device)
    _check(load().mla_quantize_fp8(_ptr(x), M, K, x.stride(0), _ptr(codes), _ptr(exps), _stream(stream)))
    return codes, exps


def mla_rope_inv_freq(rope: MlaRope, qk_rope: int, device="cuda", stream=None) -> torch.Tensor:
    """Inverse frequencies [qk_rope/2] fp64 on the device (plain, or YaRN when factor > 1)."""
    out = torch.empty(qk_rope // 2, dtype=torch.float64, device=device)
    _check(load().mla_rope_inv_freq(ctypes.byref(rope), qk_rope, out.data_ptr(), _stream(stream)))
    return out


def mla_rope_tables(positions: Optional[torch.Tensor], n: int, qk_rope: int, inv_freq=None, pos_offset: int = 0,
                    cos=None, sin=None, stream=None):
    """cos/sin [n, qk_rope/2] fp32 of (positions[t] + pos_offset) * inv_freq[i] (positions int32 on
    the device, or None for 0..n-1; inv_freq None for theta = 10000)."""
    dev = positions.device if positions is not None else (inv_freq.device if inv_freq is not None else "cuda")
    if positions is not None and (positions.dtype != torch.int32 or positions.numel() != n):
        raise MlaError("positions must be int32 [n]")
    if inv_freq is not None and (inv_freq.dtype != torch.float64 or inv_freq.numel() != qk_rope // 2):
        raise MlaError("inv_freq must be float64 [qk_rope/2]")
    cos = torch.empty((n, qk_rope // 2), dtype=torch.float32, device=dev) if cos is None else cos
    sin = torch.empty((n, qk_rope // 2), dtype=torch.float32, device=dev) if sin is None else sin
    _check(load().mla_rope_tables(n, qk_rope, _ptr(positions), pos_offset, _ptr(inv_freq), _ptr(cos), _ptr(sin),
                                  _stream(stream)))
    return cos, sin


def rope_cos_sin(positions, rope_dim: int, theta: float = 10000.0, device="cuda", inv_freq=None):
    """cos/sin tables [T, rope_dim/2] (fp32, on the device) for the given token positions,
    built by mla_rope_tables; inv_freq (fp64 device table) defaults to plain RoPE with base theta."""
    pos = torch.as_tensor(np.asarray(positions, dtype=np.int32)).to(device)
    if inv_freq is None and theta != 10000.0:
        inv_freq = mla_rope_inv_freq(rope(theta=theta), rope_dim, device)
    return mla_rope_tables(pos, pos.numel(), rope_dim, inv_freq)


def mla_qkv_prefill(cfg, w: Weights, x, cos, sin, q, k=None, v=None, kv_cache=None, slot_mapping=None, ws=None,
                    stream=None):
    """k = v = None skips the per-head K/V expansion (a chunk attended on the latent cache)."""
    act, H, dqk = _act_dtype(cfg), cfg.n_heads, cfg.qk_nope + cfg.qk_rope
    _need(x, "x", act, shape=(None, cfg.hidden))
    T = x.shape[0]
    _need_tables(cfg, cos, sin, T)
    _need(q, "q", act, numel=T * H * dqk)
    if (k is None) != (v is None):
        raise MlaError("k and v are given together or not at all")
    if k is not None:
        _need(k, "k", act, numel=T * H * dqk)
        _need(v, "v", act, numel=T * H * cfg.v_dim)
    if (kv_cache is None) != (slot_mapping is None):
        raise MlaError("kv_cache and slot_mapping are given together or not at all")
    if kv_cache is not None:
        _need_cache(cfg, kv_cache)
        _need(slot_mapping, "slot_mapping", torch.int32, numel=T)
    w.check(cfg, _FRONT + (("wkv_b",) if k is not None else ()))
    ws, nb = _ws(ws, cfg, FN_QKV_PREFILL, T, device=x.device)
    n_blocks = kv_cache.shape[0] if kv_cache is not None else 0
    _check(load().mla_qkv_prefill(ctypes.byref(cfg), ctypes.byref(w.struct), _ptr(x), T, _ptr(cos), _ptr(sin),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), _ptr(slot_mapping), n_blocks,
                                  _ptr(ws), nb, _stream(stream)))


def mla_prefill_attn(cfg, q, k, v, o, ws=None, stream=None):
    act, H, dqk = _act_dtype(cfg), cfg.n_heads, cfg.qk_nope + cfg.qk_rope
    _need(q, "q", act)
    T = q.shape[0]
    _need(q, "q", act, numel=T * H * dqk)
    _need(k, "k", act, numel=T * H * dqk)
    _need(v, "v", act, numel=T * H * cfg.v_dim)
    _need(o, "o", act, numel=T * H * cfg.v_dim)
    ws, nb = _ws(ws, cfg, FN_PREFILL_ATTN, T, device=q.device)
    _check(load().mla_prefill_attn(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), T, _ptr(o), _ptr(ws), nb,
                                   _stream(stream)))


def mla_decode_qkv_and_scatter(cfg, w: Weights, x, cos, sin, kv_cache, slot_mapping, q, ws=None, stream=None):
    act = _act_dtype(cfg)
    _need(x, "x", act, shape=(None, cfg.hidden))
    B = x.shape[0]
    _need_tables(cfg, cos, sin, B)
    _need_cache(cfg, kv_cache)
    _need(slot_mapping, "slot_mapping", torch.int32, numel=B)
    _need(q, "q", act, numel=B * cfg.n_heads * (cfg.qk_nope + cfg.qk_rope))
    w.check(cfg, _FRONT)
    ws, nb = _ws(ws, cfg, FN_DECODE_QKV, B, device=x.device)
    _check(load().mla_decode_qkv_and_scatter(ctypes.byref(cfg), ctypes.byref(w.struct), _ptr(x), B, _ptr(cos),
                                             _ptr(sin), _ptr(kv_cache), kv_cache.shape[0], _ptr(slot_mapping),
                                             _ptr(q), _ptr(ws), nb, _stream(stream)))


def mla_decode_attn_absorbed(cfg, w: Weights, q, kv_cache, block_table, context_lens, o, ws=None, stream=None):
    act = _act_dtype(cfg)
    _need(block_table, "block_table", torch.int32, shape=(None, None))
    B, max_blocks = block_table.shape
    _need(context_lens, "context_lens", torch.int32, numel=B)
    _need(q, "q", act, numel=B * cfg.n_heads * (cfg.qk_nope + cfg.qk_rope))
    _need(o, "o", act, numel=B * cfg.n_heads * cfg.v_dim)
    _need_cache(cfg, kv_cache)
    w.check(cfg, ("wkv_b",))
    ws, nb = _ws(ws, cfg, FN_DECODE_ATTN, B, max_blocks * cfg.block_size, device=q.device)
    _check(load().mla_decode_attn_absorbed(ctypes.byref(cfg), ctypes.byref(w.struct), _ptr(q), B, _ptr(kv_cache),
                                           kv_cache.shape[0], _ptr(block_table), max_blocks, _ptr(context_lens),
                                           _ptr(o), _ptr(ws), nb, _stream(stream)))


def mla_decode_attn_absorbed_noalloc(cfg, w: Weights, q, kv_cache, block_table, context_lens, o, stream=None):
    """mla_decode_attn_absorbed on the library's static scratch (no workspace argument, nothing
    allocated); calls overlapping on one GPU race."""
    act = _act_dtype(cfg)
    _need(block_table, "block_table", torch.int32, shape=(None, None))
    B, max_blocks = block_table.shape
    _need(context_lens, "context_lens", torch.int32, numel=B)
    _need(q, "q", act, numel=B * cfg.n_heads * (cfg.qk_nope + cfg.qk_rope))
    _need(o, "o", act, numel=B * cfg.n_heads * cfg.v_dim)
    _need_cache(cfg, kv_cache)
    w.check(cfg, ("wkv_b",))
    _check(load().mla_decode_attn_absorbed_noalloc(ctypes.byref(cfg), ctypes.byref(w.struct), _ptr(q), B,
                                                   _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table), max_blocks,
                                                   _ptr(context_lens), _ptr(o), _stream(stream)))


def mla_prefill_attn_paged(cfg, w: Weights, q, kv_cache, block_table, prefix_len: int, o, ws=None, stream=None):
    """Chunk of T = q.shape[0] tokens at positions prefix_len.. over one sequence's cache
    (block_table int32 [max_blocks])."""
    act = _act_dtype(cfg)
    _need(q, "q", act)
    _need(block_table, "block_table", torch.int32, shape=(None,))
    T, max_blocks = q.shape[0], block_table.numel()
    _need(q, "q", act, numel=T * cfg.n_heads * (cfg.qk_nope + cfg.qk_rope))
    _need(o, "o", act, numel=T * cfg.n_heads * cfg.v_dim)
    _need_cache(cfg, kv_cache)
    w.check(cfg, ("wkv_b",))
    ws, nb = _ws(ws, cfg, FN_PREFILL_ATTN_PAGED, T, max_blocks * cfg.block_size, device=q.device)
    _check(load().mla_prefill_attn_paged(ctypes.byref(cfg), ctypes.byref(w.struct), _ptr(q), T, _ptr(kv_cache),
                                         kv_cache.shape[0], _ptr(block_table), max_blocks, int(prefix_len), _ptr(o),
                                         _ptr(ws), nb, _stream(stream)))


def mla_out_proj(cfg, w: Weights, o, y, ws=None, stream=None):
    act = _act_dtype(cfg)
    _need(o, "o", act)
    M = o.shape[0]
    _need(o, "o", act, numel=M * cfg.n_heads * cfg.v_dim)
    _need(y, "y", act, shape=(M, cfg.hidden))
    w.check(cfg, ("wo",))
    ws, nb = _ws(ws, cfg, FN_OUT_PROJ, M, device=o.device)
    _check(load().mla_out_proj(ctypes.byref(cfg), ctypes.byref(w.struct), _ptr(o.reshape(M, -1)), M, _ptr(y),
                               _ptr(ws), nb, _stream(stream)))
