"""CPU oracle for exact scaled dot-product attention (fp64, numpy).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never links, imports or calls it, and this package
imports nothing from the HIP side: the two share no code.  Inputs come from the
seeded generators in ``workloads`` (which hold none of the method's arithmetic).

Sources (the three web pages this method is described on):

* "Module 08: FlashAttention and Memory-Efficient Kernels" (backend-roadmap),
  sections "Where the time goes in standard attention", "Tiling and the online
  softmax", "The backward pass: recompute instead of store", Steps 1, 3 and 6.
* "FlashAttention in Triton: A Tile-by-Tile Walkthrough" (riteshyadav.xyz),
  sections "First, what does attention actually do?" and "How can softmax work a
  tile at a time?" (the three-key worked example).
* "FlashAttention-style kernel" (roadmapper), sections "The loop", "Causal
  masking" and "Things that break".

Contents:

* :mod:`oracle.definition` - the plain definition: S = scale*Q K^T, masked row
  softmax P, O = P V, LSE = m + log(sum exp(S - m)).  Materialises S and P.
* :mod:`oracle.online` - the streaming (online-softmax) recurrence written out
  step by step, used only to pin the recurrence itself against the definition
  and the pages' printed trace, plus the failure modes the pages name.
* :mod:`oracle.backward` - gradients of the definition (dQ, dK, dV) and the
  rebuild of P from the saved LSE, in fp64.
* :mod:`oracle.split` - attention over key chunks and the merge of the partial
  (O, LSE) pairs by the concatenation algebra.

Every function here has at least one pin in ``tests/test_oracle_*.py``; none is
"parity unpinned".
"""

from .definition import attention, attention_rows, visible_mask, scale_as_kernel  # noqa: F401
from .online import online_softmax_trace, tiled_attention  # noqa: F401
from .backward import attention_bwd, head_bwd, recompute_p  # noqa: F401
from .split import merge_partials, partial_attention, split_attention  # noqa: F401
