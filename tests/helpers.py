"""Shared plumbing of the GPU parity tests: device copies of synth inputs, the
library config of a workload, and the error metric of the parity bar."""
import numpy as np
import pytest
import torch

import synth
from synth import torch_io

# max|gpu - oracle| / max|oracle| per output tensor (fp32 config: 1e-4; bf16 / fp8: 2e-2)
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite GPU output"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def assert_close(got, ref, kind, what):
    e = rel_err(got, ref)
    print(f"  {what}: max-rel-err {e:.3e} (tol {TOL[kind]:.0e})", flush=True)
    assert e <= TOL[kind], f"{what}: {e:.3e} > {TOL[kind]}"


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
