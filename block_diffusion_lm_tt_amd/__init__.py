"""MI355X-native hot path of one block-wise diffusion decoding step (Nemotron-TwoTower).

The computation lives in libtt.so (HIP kernels for gfx950 behind a C-ABI, include/tt.h);
this package is its Python binding plus the seeded synthetic workloads.
"""
from ._lib import (TTError, header_symbols, lib, profile_enable, profile_read, profile_reset,  # noqa: F401
                   tt_adaln_gate, tt_adaln_modulate, tt_block_denoise_attn, tt_block_denoise_attn_workspace,
                   tt_commit, tt_commit_workspace, tt_ctx_append, tt_lmhead_commit, tt_lmhead_commit_workspace,
                   tt_lmhead_weight_bound, tt_mamba2_seeded_scan)

__all__ = ["tt_block_denoise_attn", "tt_commit", "tt_ctx_append", "tt_lmhead_commit",
           "tt_mamba2_seeded_scan", "tt_adaln_modulate", "tt_adaln_gate",
           "tt_block_denoise_attn_workspace", "tt_commit_workspace", "tt_lmhead_commit_workspace",
           "tt_lmhead_weight_bound",
           "TTError", "profile_enable", "profile_reset", "profile_read", "lib", "header_symbols"]
