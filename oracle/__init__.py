"""CPU oracle for Mixture-of-Gaussians (Iceberg) decode attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (the HIP library and its Python binding) never
does, and this package imports nothing from the product.

Everything here is plain NumPy in float64, written to be read against the
pages, step by step. See ``oracle/mog.py`` for the algorithm and the readings
taken where the pages are silent.
"""

from .mog import (  # noqa: F401
    GOLDEN_GAMMA,
    splitmix64,
    unit_state,
    sub_state,
    forgy_ids,
    ceil_sqrt,
    ceil_log2,
    unit_dims,
    nearest_centroid,
    partition_sse,
    lloyd,
    group_stats,
    group_log_mass,
    bf16_round,
    decode_statistics,
    top_by_score,
    UnitLayout,
    build_unit,
    layout_from_assignment,
    fold_tokens,
    positive_features,
    with_feature_summaries,
    fm_log_mass,
    shared_selection,
    decode_unit,
    dense_attention,
    decode_batch,
    dense_batch,
)
