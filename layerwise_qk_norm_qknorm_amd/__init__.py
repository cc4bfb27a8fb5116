"""Layerwise QK-Norm for MI355X (gfx950): HIP kernels behind a small C ABI.

The compute lives in ``libqknorm.so`` (built from ``csrc/``); this package is
argument marshalling only. Importing it does not load the library; the first
call does, and raises if the library has not been built.
"""

from .binding import (  # noqa: F401
    PreparedCall,
    QKNormError,
    abi_version,
    describe_headwise_plan,
    describe_plan,
    library_path,
    load_library,
    qknorm_apply_with_stats,
    qknorm_fused,
    qknorm_headwise,
    qknorm_partial_stats,
    prepare_apply_with_stats,
    prepare_fused,
    prepare_headwise,
    prepare_partial_stats,
)
