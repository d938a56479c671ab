"""decode_attention_shared_hw_amd — Hogwild! concurrent-attention decode on MI355X.

The compute lives in libhogwild_attn.so (hand-written HIP for gfx950, C ABI in
include/hogwild_attn.h).  `hogwild_attn` is its ctypes binding; `layout` maps
logical K/V to the pool's tile layout; `workloads` generates seeded synthetic
inputs.  Submodules load lazily so that importing the package needs no GPU.
"""
__all__ = ["hogwild_attn", "layout", "workloads", "build"]
