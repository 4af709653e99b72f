"""CPU fp64 oracle for attention over a flat, slot-addressed KV pool.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``paged_kv_attention_12_amd``) and never imports it.

Every function is a plain, unblocked restatement of what the AstrAI pages say
is computed (see the citations on each function).  Floating point is float64
throughout; inputs of any float dtype are upcast exactly.
"""

from .attention import (  # noqa: F401
    NEG_INF,
    attend,
    build_step,
    decode,
    decode_pairs,
    decode_split,
    kv_store,
    merge_partials,
    prefill,
    prefill_rows,
    split_partial,
    validate_step,
)
from .rope import (  # noqa: F401
    round_to_bf16, rope_kv_store, rope_rotate, rope_rotate_tail, to_dtype)
from . import pages  # noqa: F401,E402  (pools of page_size > 1 tokens)
