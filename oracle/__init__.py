"""fp64 CPU oracle for the speculative verification step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing) and it
imports nothing from the library's package.

What it computes, and from which passage:

* ``attention`` -- the target model's attention for the verify queries over
  the long-context KV cache plus the masked draft block, written as the plain
  unsplit softmax-attention definition.  The hybrid tree attention of the
  LongSpec summary (gist.science, "LongSpec", section 2.3 "Fast Tree
  Attention") splits this into an unmasked history part and a masked
  speculative part merged by log-sum-exp; that split reaches the same result
  up to rounding order, so the oracle is the definition itself.  The
  log-sum-exp merge of partial results is provided separately
  (``lse_merge_ref``) to pin the split identity.

* ``rapid`` -- RAPID's acceptance step (RAPID blog, leeon-k.github.io,
  section 2.1 "Background: speculative decoding", section 2.3 "RAG drafter",
  section 2.4 "Retrieval-augmented target distribution"; abeam.tech RAPID
  article, "Key idea 1: Retrieval-Augmented Target Distribution"), taken
  step by step with caller-supplied uniforms: p = softmax(z/T),
  q = softmax(y/T), p_hat = softmax(z/T + eta*(q - p)), the test
  r <= min(1, p_hat/q) with a first-reject cut, and inverse-CDF sampling
  from norm(max(p_hat - q, 0)) at the first rejection (or from the target
  distribution of the last row when every draft is accepted).

All floating point is IEEE binary64.  bf16 inputs arrive as raw uint16 bit
patterns and are widened exactly; fp32 inputs are widened exactly.

* ``window`` -- the drafter's sliding-window self-attention with attention-
  sink anchors over its constant-size ring cache (LongSpec summary, sections
  2.1 and 2.2), written as the definition over the visible positions.

* ``tree`` -- acceptance over a draft tree: a rule from outside the pages
  (they verify trees only as attention), recursive rejection among sibling
  candidates with p_hat as the target, which reduces to ``rapid`` on a chain.

Blog section 2.4 also prints a tail-preserving adjustment of p_hat and a
different residual; both are available as options of ``rapid_accept_ref``
(off by default) with the readings stated in ``rapid``.

Every function is pinned by ``-m "not gpu"`` tests against facts fixed
outside this package (library routines, closed forms, brute force, the
fixed points the pages state, exact enumeration and Monte-Carlo of the
sampling law).  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    block_visibility,
    attn_ref,
    attn_keys_ref,
    lse_merge_ref,
)
from .window import (  # noqa: F401
    ring_slot,
    window_attn_ref,
    window_positions,
)
from .rapid import (  # noqa: F401
    softmax_ref,
    target_probs,
    draft_probs,
    retrieval_augmented_target,
    inverse_cdf_ref,
    rapid_accept_ref,
    tail_preserve_ref,
)
from .tree import (  # noqa: F401
    rapid_tree_accept_ref,
    residual_sequence,
    tree_children,
)
