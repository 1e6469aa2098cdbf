"""fp64 CPU oracle for the block-denoise attention, the confidence commit (also behind the
LM head), the context cache update after a commit, and the denoiser's Mamba-2 scan from a
seeded state and adaLN-single time modulation.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library or its binding.
"""
from .ttref import (ttref_adaln_gate, ttref_adaln_modulate, ttref_block_denoise_attn,  # noqa: F401
                    ttref_commit, ttref_ctx_append, ttref_decode, ttref_lmhead_commit, ttref_mamba2_scan,
                    ttref_threads, lib_path)
