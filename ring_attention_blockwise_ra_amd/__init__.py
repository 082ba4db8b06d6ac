"""MI355X-native (gfx950) Ring Attention per-device step.

The compute path is the HIP library libra_amd.so (C ABI in include/ra.h);
``ring_attention_blockwise_ra_amd.binding`` marshals torch tensors to it.
Importing this package loads nothing; the library is loaded on first use and
its absence is an error, never a fallback.
"""

_BINDING_NAMES = (
    "ra_block_attn_partial", "ra_merge_partials", "ra_finalize", "ra_ring_workspace_bytes",
    "ra_ring_fwd", "ra_tile_class_host", "ra_tile_classes_host", "ra_tile_classes_device",
    "ra_attn_bwd_delta", "ra_block_attn_bwd", "ra_ring_bwd_workspace_bytes", "ra_ring_bwd",
    "ra_rope_apply", "make_problem", "RaError", "RaProblem", "lib",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
