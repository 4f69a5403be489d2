"""MI355X-native multi-head latent attention (MLA) hot path.

The computation lives in libmla.so (hand-written HIP kernels for gfx950); this
package only marshals torch tensors into its C ABI (see ``binding``)."""
from .binding import (MLA_BF16, MLA_F32, MLA_FP8_E4M3, MlaConfig, MlaError, MlaRope, Weights, config, load,
                      mla_decode_attn_absorbed, mla_decode_attn_absorbed_noalloc, mla_decode_qkv_and_scatter, mla_out_proj, mla_prefill_attn,
                      mla_prefill_attn_paged, mla_qkv_prefill, mla_quantize_fp8, mla_rope_inv_freq, mla_rope_tables, rope, rope_cos_sin, workspace,
                      workspace_size)

__all__ = ["MLA_BF16", "MLA_F32", "MLA_FP8_E4M3", "MlaConfig", "MlaError", "MlaRope", "Weights", "config", "load",
           "mla_decode_attn_absorbed", "mla_decode_attn_absorbed_noalloc", "mla_decode_qkv_and_scatter", "mla_out_proj", "mla_prefill_attn",
           "mla_prefill_attn_paged", "mla_qkv_prefill", "mla_quantize_fp8", "mla_rope_inv_freq", "mla_rope_tables", "rope", "rope_cos_sin", "workspace",
           "workspace_size"]
