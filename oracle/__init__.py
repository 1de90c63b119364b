"""FP64 CPU oracle for exact softmax attention, split-KV decode and row softmax.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library under ``online_softmax_fa2_amd``
and its Python binding) never imports it, and this package imports nothing
from the product path: the two share no code.

Modules
  attention -- the direct definition of softmax attention (masked), decode.
  backward  -- the gradients dQ, dK, dV of masked softmax attention, and a
               first-order bound on their rounding error (a tolerance).
  softmax   -- the direct definition of row softmax and its top-k.
  quantized -- the error model of FP8 (e4m3) attention against the exact
               attention of the dequantized inputs (a tolerance).
  models    -- the pages' streaming algorithms (per-element (m, d) update,
               the associative merge, the single-query and query-tile
               blockwise recurrences, split-KV), written from their
               equations; used only to test the pages' claims against the
               direct definitions, including planted-mistake variants.

Every function states the passage of the pages it follows.  The pages are
cited by title: "Derive online softmax, prove it is exact" (the single-query
derivation, the backward pass's recomputation from the log-sum-exp),
"Online softmax for a whole query tile, matrix form" (the tile form, masks,
the guard, FA2's deferred division) and "Online softmax" (the
article on Milakov and Gimelshein's online normalizer: Steps 1-4, the worked
example, trade-offs).

Parity pins: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` against values printed on the pages, closed forms,
invariants and brute force.  No function is "parity unpinned".
"""

from .attention import attention_ref, decode_ref, visible_mask, visible_count  # noqa: F401
from .softmax import softmax_ref, topk_ref  # noqa: F401
from .quantized import attention_fp8_error_bound, attention_fp8_error_model  # noqa: F401
from .backward import attention_bwd_ref, attention_bwd_delta, attention_bwd_error_bound  # noqa: F401
