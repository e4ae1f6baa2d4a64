"""MI355X-native MoE dispatch layout, dispatch and combine.

The work runs in hand-written HIP kernels for gfx950 behind the C ABI declared in
``include/moe_dispatch.h`` (library ``libmoedl.so``).  ``moedl`` is the thin Python
binding over it (argument marshalling only); ``workloads`` draws seeded synthetic
inputs.
"""
__all__ = ["moedl", "workloads"]
