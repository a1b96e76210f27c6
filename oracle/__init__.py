"""Oracle for ragged paged attention and the paged KV-cache write.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``ragged_paged_kv_amd``) never imports it and shares no code
with it; the two meet only in the seeded input generator ``synth``.

Plain, slow, obviously correct CPU code in numpy float64. Each function cites
the passage of the pages it restates. Pins (tests that tie these functions to
something other than themselves) live in ``tests/test_oracle_*.py``; every
function here is pinned, none is "parity unpinned" as a function, but no page
prints an attention output value, so attention numbers are pinned by closed
forms, a library special case, a brute-force masked formulation and
invariants rather than by printed values.
"""
from .attention import (  # noqa: F401
    bf16_to_f64,
    slot_mapping,
    cache_write,
    unpage,
    paged_attention,
    split_partials,
    merge_partials,
    within_tolerance,
    ATOL,
    RTOL,
)
from .packing import (  # noqa: F401
    occupancy,
    rectangle_count,
    prompt_among_decodes,
    block_layout,
    pack_ragged,
    SMALLEST_BLOCK,
)
