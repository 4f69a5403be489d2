"""Shared plumbing of the GPU parity tests: device copies of synth inputs, the
library config of a workload, and the error metrics of the parity bar."""
import numpy as np
import pytest
import torch

import synth
from synth import torch_io

# Parity bar (fp32 config: 1e-4; bf16 / fp8: 2e-2), checked two ways:
#   per tensor:  max|gpu - oracle| / max|oracle| over the whole output;
#   per row:     the same ratio within each leading index (a query row, a token, a sequence),
#                so that rows of small magnitude (late causal queries, short sequences) are held
#                to the bar relative to their own size rather than to the tensor's largest row.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite GPU output"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def row_rel_err(got: np.ndarray, ref: np.ndarray):
    """max over leading indices i of max|got[i] - ref[i]| / max|ref[i]|; returns (error, worst i).
    A 1-D array is one row."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.ndim == 1:
        got, ref = got[None], ref[None]
    assert np.isfinite(got).all(), "non-finite GPU output"
    n = got.shape[0]
    d = np.max(np.abs(got - ref).reshape(n, -1), axis=1)
    m = np.maximum(np.max(np.abs(ref).reshape(n, -1), axis=1), 1e-30)
    e = d / m
    i = int(np.argmax(e))
    return float(e[i]), i


def assert_close(got, ref, kind, what, rows=None):
    """Both gates; `rows` names the leading indices (for the message: sampled row numbers)."""
    e = rel_err(got, ref)
    er, i = row_rel_err(got, ref)
    label = i if rows is None else int(np.asarray(rows)[i])
    print(f"  {what}: max-rel-err {e:.3e}, worst row {er:.3e} (row {label}) (tol {TOL[kind]:.0e})", flush=True)
    assert e <= TOL[kind], f"{what}: {e:.3e} > {TOL[kind]}"
    assert er <= TOL[kind], f"{what}: row {label}: {er:.3e} > {TOL[kind]}"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def lib_config(shape: synth.MlaShape):
    import head_latent_attention_amd as mla
    return mla.config(shape.hidden, shape.n_heads, shape.q_lora_rank, shape.kv_lora_rank, shape.qk_nope,
                      shape.qk_rope, shape.v_dim, act=shape.act, weight=shape.weight,
                      block_size=shape.block_size, norm_eps=shape.norm_eps, act_quant=shape.act_quant)


def device_weights(host: dict):
    import head_latent_attention_amd as mla
    tens = {k: torch_io.to_device(v) for k, v in host.items()}
    scales = {k: torch_io.scale_to_device(v) for k, v in host.items() if v.scale is not None}
    return mla.Weights(tens, scales)


def sentinel_cache(shape: synth.MlaShape, n_blocks: int) -> torch.Tensor:
    """A cache whose every element holds a sentinel bit pattern (fp32 12345.0 / bf16 0x4640)."""
    if shape.act == "f32":
        return torch.full((n_blocks, 1, shape.block_size, shape.row), 12345.0, dtype=torch.float32, device="cuda")
    return torch.full((n_blocks, 1, shape.block_size, shape.row), 12345.0, dtype=torch.bfloat16, device="cuda")
