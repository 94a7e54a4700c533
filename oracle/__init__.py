"""Plain CPU oracle of the OWQ hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (``mixed_precision_weight_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``owq_oracle.c`` (plain C, fp64 sums, IEEE fp32 steps,
built without FMA contraction); this module is argument marshalling over numpy
arrays plus ``build()``.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    f16_to_f64,
    f32_to_f16,
    qparams,
    code,
    hessian_diag,
    rtn_col_err,
    calibrate_score,
    select_weak,
    pack,
    pack_search,
    pack_storage,
    pack_grouped,
    linear_grouped_rows,
    optq_factor,
    optq_pack,
    f64_to_f16,
    linear_storage_rows,
    search_qparams,
    SEARCH_STEPS,
    unpack_codes,
    linear_pairs,
    linear_full,
    linear_rows,
    linear_backward,
    effective_bits,
)
