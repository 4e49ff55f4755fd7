"""Shard-invariant exact softmax attention and deterministic cross-entropy for
AMD MI355X (gfx950), behind the C ABI in include/det_attn.h.

    from bitwise_deterministic_exact_pass1_amd import det_attn, det_attn_sharded
    from bitwise_deterministic_exact_pass1_amd import cross_entropy as dce

The submodules load the compiled library lazily; `workloads` (seeded inputs)
imports without it.
"""
from __future__ import annotations

__all__ = ["det_attn", "det_attn_sharded", "det_attn_composed", "rowmax", "accumulate", "combine_rowmax",
           "combine_digits", "finalize", "default_scale"]


def __getattr__(name):
    if name in __all__:
        from . import attention
        return getattr(attention, name)
    raise AttributeError(name)
