"""MI355X-native MoE layer with affinity-aware token dispatch.

The compute path is the HIP library ``libmoe.so`` (gfx950) behind a C ABI
(include/moe.h); ``token_routing_shuffle_amd.moe`` is its thin ctypes binding.
``workload`` draws seeded synthetic layers; ``offline`` builds the offline
tables (placement-ordered weights, token->group lookup table).
"""
__all__ = ["moe", "workload", "offline"]
