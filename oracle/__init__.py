"""CPU fp64 oracle for blockwise causal attention, its backward and the LSE merge.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, calls or links anything here; only the tests, the
``smoke()`` check and the bench's CPU-baseline leg do.  The oracle shares no
code with the HIP path: it derives positions, masks and every formula itself.

What it computes is the plain definition of masked softmax attention (the
method only rearranges this computation exactly: tiling, online rescaling and
the merge of partial results over key blocks change the rounding order and
nothing else).  Sources for the method:

* EasyContext core-technology page (hotelren.com), section 1 "sequence
  parallelism" (ring attention splits a sequence over GPUs) and section 2
  "Flash Attention optimisation" (tiling plus recomputation instead of a stored
  attention matrix; the forward and backward kernels it calls).
* EasyContext 200-line training-script walkthrough (mlqm.cn), section on model
  preparation and parallel strategies (the zigzag ring mode that interleaves
  tokens across ranks).
* EasyContext "1M tokens with minimal resources" page (cn486.com), usage code
  (each rank receives its local shard together with its local position ids).
* The fused cross-entropy with in-place backward that the training step uses
  (EasyContext ZeRO-3 offload page, kwkr.cn, section on advanced optimisation
  combined with other techniques, item 1; cn486.com page, the summary of the
  training script's technology stack): ``xent.py``.
* The rotary position embedding whose base the pages raise for long contexts
  (hotelren.com page, further optimisations; mlqm.cn walkthrough, the
  rope-theta option; kwkr.cn page, training script and advanced optimisation
  item 2; cn486.com page, training strategy): ``rope.py``.

Where the pages are silent (no formula, layout or mask rule is printed on any
of them) the reading taken is stated next to the function that uses it.

Functions are pinned by the ``-m "not gpu"`` tests: pure-Python brute force on
tiny inputs, torch fp64 autograd, finite differences, closed forms, exact
invariants (key-split merge, zigzag reassembly) and hand-derived fixtures.
"""
from .attention import (  # noqa: F401
    allowed_mask, allowed_sums, attn_fwd, attn_bwd, lse_merge, attn_fwd_heads, attn_bwd_heads,
)
from .zigzag import zigzag_positions, ring_source, chunk_positions  # noqa: F401
from .xent import xent_fwd_bwd  # noqa: F401
from .rope import round_bf16, attn_bwd_rope, attn_bwd_rope_heads  # noqa: F401  (oracle.rope stays the module; its rope() is oracle.rope.rope)
