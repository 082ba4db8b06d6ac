"""CPU oracle for one device's share of Ring Attention (test infrastructure).

This package is test infrastructure only. It may be imported by the test
suite, by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py`` -- never by the product path under
``ring_attention_blockwise_ra_amd/``. It shares no code with the HIP path.
"""

from .ring_oracle import (  # noqa: F401
    SKIP, PARTIAL, FULL,
    default_scale,
    kv_head_of,
    global_positions,
    ring_order,
    naive_attention,
    naive_attention_rows,
    block_partial,
    empty_partial,
    merge_partials,
    finalize,
    ring_share,
    ring_share_literal,
    tile_classes_bruteforce,
    visible_pairs_bruteforce,
    visible_pairs_closed_form,
    counted_flops,
)
