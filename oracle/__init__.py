"""CPU oracle of KV-cache importance scoring and compaction after prefill.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything here.  The
library (``kv_cache_compression_softmax_amd``) never imports it and shares no
code with it: the two meet only on the seeded inputs of
``kv_cache_compression_softmax_amd.synth``.

The oracle is plain numpy in float64, written from the pages' definitions:
  * ``infokv``    InfoKV's score S = alpha*A + (1-alpha)*softmax(D*H), budgets,
                  selection, gather, decode attention and RECAS's dropped-mass
                  bound;
  * ``selkv``     SelKV's VATP + GQA-union selection, bucket routing, soft
                  cosine gate, gated merge and log-ratio compensation;
  * ``recas``     RECAS's active-set decoding (sparse score, top-K_t active
                  set, attention over it);
  * ``precision`` exact bf16 <-> float64 conversions.

Pins (closed forms, invariants, library special cases, brute force) live in
``tests/test_oracle_*.py``.  Absolute values at the large Llama-shaped sizes
are pinned only through those invariants and the shared code; the readings the
pages leave open (group union, gated ratio, merge target) are choices no page
number confirms.
"""
from . import infokv, precision, recas, selkv  # noqa: F401
