"""fp64 CPU oracle for paged-KV decode attention. TEST INFRASTRUCTURE ONLY.

Only the tests under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The product path (``paged_kv_decode_xs_amd``) never does, and this
package never imports the product path. The two share no code. Their only
common input is the seeded generator in ``workloads``, which holds none of
the attention arithmetic.

Contents:

* ``paged_attention``: the plain definition, written out in fp64 with numpy:
  the decode-step append, the gather through the block table, GQA
  softmax(q K^T * scale) V, per-partition softmax statistics with their
  log-sum-exp merge, and the naive causal attention it must agree with at the
  last position.
* ``sinks_window``: the same decode with per-head attention sinks and a
  sliding window, unsplit and split (the sink joins once, in the merge).
* ``prefill``: the chunked-prefill step over the pools: multi-token append from a start
  position, then causal (bottom-right aligned) attention of the chunk's queries, also with
  per-head sinks and a sliding window.
* ``swap``: KV block swap-out / swap-in between the pools and host swap space
  (bit copies of whole blocks, list-driven).
* ``brute_force``: the definitions again, in Python ``decimal`` at
  40 digits over flat offsets, for tiny inputs only.

Every function is pinned by the CPU tests in ``tests/test_oracle_*.py``
against facts the pages and the mathematics fix (closed forms, invariants, a
library routine on the contiguous special case, the brute force, and a
hand-derived fixture). No function here is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    decode_values,
    kv_append,
    gather_kv,
    paged_decode_attention,
    attention_weights,
    partition_stats,
    lse_merge,
    split_paged_decode_attention,
    naive_causal_attention,
)
from .prefill import kv_append_chunk, paged_prefill_attention, paged_prefill_attention_sinks  # noqa: F401
from .sinks_window import (  # noqa: F401
    window_start,
    paged_decode_attention_sinks,
    partition_stats_window,
    lse_merge_sink,
    split_paged_decode_attention_sinks,
)
