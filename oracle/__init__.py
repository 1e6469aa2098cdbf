"""fp64 CPU oracle for the block-denoise attention and the confidence commit.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library or its binding.
"""
from .ttref import ttref_block_denoise_attn, ttref_commit, ttref_decode, ttref_threads, lib_path  # noqa: F401
