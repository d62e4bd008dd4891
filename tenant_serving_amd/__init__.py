"""MI355X-native BitDelta: fused 1-bit-delta linear and compression (gfx950 HIP).

The compute lives in libbitdelta.so (hand-written HIP kernels behind a C ABI,
``include/bitdelta.h``); this package is its thin ctypes binding plus the
seeded synthetic-input generators.  There is no CPU fallback.
"""

from .bitdelta import (  # noqa: F401
    BD_ALPHA_PER_MATRIX,
    BD_ALPHA_PER_ROW,
    BD_MAX_VARIANTS,
    BitDeltaError,
    bd_compress,
    bd_compress_pair,
    bd_linear,
    bd_linear_bf16,
    bd_linear_grouped,
    bd_linear_grouped_noalloc,
    bd_linear_grouped_plan,
    bd_linear_path,
    library,
)
from .cache import Busy, bd_cache  # noqa: F401
