"""fp64 CPU oracle for the block-denoise attention, the confidence commit (also behind the
LM head) and the context cache update after a commit.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library or its binding.
"""
from .ttref import (ttref_block_denoise_attn, ttref_commit, ttref_ctx_append, ttref_decode,  # noqa: F401
                    ttref_lmhead_commit, ttref_threads, lib_path)
