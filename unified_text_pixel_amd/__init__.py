"""Hybrid-masked joint self-attention for unified text+pixel image transformers on
AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI (include/ha_attn.h), with a
ctypes binding (binding.py) and a torch-facing layer (api.py)."""
from .binding import (EXPORTS, HAError, AttnDesc, PrologueDesc, load_library, ha_abi_version,
                      ha_last_error, ha_rope_table_fill, ha_q_prescale, ha_tile_shape, ha_classify_tiles,
                      ha_qk_prologue, ha_attn_workspace_bytes, ha_attn_fwd_planned, ha_attn_fwd,
                      ha_attn_fwd_lse, ha_attn_bwd_workspace_bytes, ha_attn_bwd, ha_qk_prologue_from,
                      ha_attn_fwd_planned_from, ha_qkv_prologue, ha_attn_fwd_static)

__all__ = ["EXPORTS", "HAError", "AttnDesc", "PrologueDesc", "load_library", "ha_abi_version",
           "ha_last_error", "ha_rope_table_fill", "ha_q_prescale", "ha_tile_shape", "ha_classify_tiles",
           "ha_qk_prologue", "ha_attn_workspace_bytes", "ha_attn_fwd_planned", "ha_attn_fwd",
           "ha_attn_fwd_lse", "ha_attn_bwd_workspace_bytes", "ha_attn_bwd", "ha_qk_prologue_from",
           "ha_attn_fwd_planned_from", "ha_qkv_prologue", "ha_attn_fwd_static"]
