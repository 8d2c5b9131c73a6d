"""Plain, slow CPU oracle for paged KV-cache attention (fp64 NumPy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library: no kernels, headers, helpers, tables or constants.

Citation key (the pages are AstrAI commit pages; a "bullet" is one line of the
commit message shown on that page):
  P1  commit 398e8a3e, page for tests/inference/test_cache.py
  P2  commit 8e39d9d8, page for astrai/inference/workspace.py
  P3  commit f8d9ab34, page for astrai/trainer/rollout.py
  P4  commit e58a728b, page for docs/developer/architecture.md

Pins: every function below is checked by ``tests/test_oracle_*.py`` against
something other than itself (a library routine, a closed form, an invariant,
or a hand-derived fixture in ``tests/golden/``). Functions whose semantics rest
only on a reading of the pages, not on anything the pages fix, say so.
"""

from .paged_attention import (  # noqa: F401
    kv_store,
    kv_indptr,
    decode_locations,
    prefill_locations,
    split_plan,
    split_ranges,
    decode_attention,
    decode_split_partials,
    lse_merge,
    prefill_attention,
    gathered_kv,
    rope_pairs,
    apply_rope,
    rope_kv_store,
)
from .fp8_kv import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    quantize,
    dequantize,
    kv_store_fp8,
    decode_attention_fp8,
    prefill_attention_fp8,
    rope_fp32,
    rope_kv_store_fp8,
)
