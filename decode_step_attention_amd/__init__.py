"""Fused decode-step masked multi-head attention over a KV cache for AMD
MI355X (gfx950).

The computation lives in libftm.so (C ABI in include/ftm.h); ``ftm`` is its
Python binding and ``workloads`` the seeded synthetic inputs.  Import
``decode_step_attention_amd.ftm`` to load the library.
"""
__all__ = ["ftm", "workloads"]
