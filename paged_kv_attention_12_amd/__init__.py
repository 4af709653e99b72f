"""MI355X (gfx950) attention over a flat, slot-addressed KV pool.

The compute lives in libpkv.so (hand-written HIP kernels behind the C ABI in
include/pkv.h); this package only marshals arguments to it.
"""

from .binding import (  # noqa: F401
    PKV_BF16,
    PKV_F32,
    PkvError,
    load,
    make_pool,
    make_step,
    pkv_build_step,
    pkv_decode_pick_splits,
    pkv_decode_workspace_bytes,
    pkv_kv_store,
    pkv_paged_decode,
    pkv_paged_decode_merge,
    pkv_paged_prefill,
    pkv_validate_step,
)
from .api import DeviceStep, decode_step, prefill_step  # noqa: F401
