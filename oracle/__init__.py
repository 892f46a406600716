"""fp64 CPU oracle for exact attention: TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously correct statement of what the GPU library
computes.  Only the test suite, the smoke check and the bench's CPU-baseline leg
may import it.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here, and this package imports nothing from the
product path: the two share no code.  Inputs reach both sides from the seeded
generators, which hold none of the method's arithmetic.

Sources (cited by page title and section throughout):

* "精读笔记 08：FlashAttention" -- close-reading notes on the FlashAttention
  paper (llm-papers-study.pages.dev), called *FA notes* below.  Used: §2.1
  (standard attention, Algorithm 0), §3.1 (online softmax merge rule), §3.2
  (tiled forward pseudocode), §3.3 (recomputation), §3.5 (IO complexity).
* "S12 FlashAttention" -- chapter of an LLM-inference course
  (llminference.xinbetween.com/zh/s12), called *S12* below.  Used: the
  "core idea" NumPy recurrence, the "how it works" recurrence box, the paged
  "implement it" loop, the NaN box, the production-practice paragraph on
  paged + GQA decode, and exercises 1-2.
* "FlashAttention IO-aware explained" (shandesong.com), called *IO explainer*.

Modules:

* ``reference`` -- the plain definitions: forward, backward, paged decode.
* ``online``    -- the method's own loops, written from the pages: the KV-outer
  tiled forward of FA notes §3.2, the S12 deferred-normalisation recurrence,
  the split-K (m, l, o) merge of S12 exercise 1, and the S12 paged loop.
* ``brute``     -- pure-Python scalar loops for tiny inputs.
* ``varlen``    -- packed variable-length batches (block-diagonal visibility),
  forward and backward, and prefill of packed new tokens against a paged
  cache.
* ``sparse``    -- block-sparse attention (exact under a block mask), forward
  and backward.
* ``dropout``   -- dropout on the probability matrix (FA notes §2.1 / §3.4)
  with a counter-based generator (Philox4x32-10), forward and backward.

Pin status: every public function here is pinned by the CPU tests against
closed forms, invariants, brute force or finite differences; none is marked
"parity unpinned".
"""

from .reference import (  # noqa: F401
    attention_fwd,
    attention_bwd,
    decode_paged,
    k_cache_rows,
    visible_mask,
)
from .online import (  # noqa: F401
    M_GUARD,
    kv_outer_tiled,
    online_rows,
    split_merge,
    merge_triples,
    paged_online,
)
from .brute import brute_fwd  # noqa: F401
from .dropout import (  # noqa: F401
    attention_bwd_dropout,
    attention_fwd_dropout,
    dropout_keep,
    dropout_threshold,
    philox4x32_10,
)
from .sparse import (  # noqa: F401
    attention_bwd_block_sparse,
    attention_fwd_block_sparse,
    block_sparse_visible,
)
from .varlen import (  # noqa: F401
    attention_bwd_varlen,
    attention_fwd_varlen,
    prefill_paged,
    varlen_visible,
)
