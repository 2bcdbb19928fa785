"""fp64 CPU oracle of the paged-KV, variable-length attention step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP path is checked against.  Only the test suite, the
smoke check and the bench's CPU-baseline leg may import it; the product path
(the C-ABI library and its Python binding) never does, and shares no code with
it.  It uses numpy (and, in one pin, torch's CPU attention routine) only.

What it defines, with the passages it follows (pages are cited by title and
section; "Inside vLLM summary" is the techfeed.io article summarising
"Inside vLLM: Anatomy of a High-Throughput LLM Inference System"):

  * ``RefBlockPool`` -- the block allocator: 16-token blocks, ceil(tokens/16)
    blocks per request, blocks taken from the head of ``free_block_queue`` into
    ``req_to_blocks`` (Inside vLLM summary, "PagedAttentionの仕組み"); shared
    prefix blocks with reference counts (same page, "高度な機能群", Prefix
    Caching); blocks handed back on release (the engr-sng explainer of the same
    article, paragraph on Paging Attention).
  * ``ref_reshape_and_cache`` -- the step's new K/V rows written into their cache
    slots, bit for bit.
  * ``ref_attention_paged`` / ``ref_attention_dense`` -- causal attention of
    each sequence over its own tokens only, reading K/V through the block table
    or from contiguous per-sequence arrays (Inside vLLM summary,
    "PagedAttentionの仕組み", flattened super-sequence with positions and mask).
  * ``ref_bruteforce`` -- pure-Python loops with an explicit 0/1 mask over every
    token of the super-sequence; tiny inputs only.

Readings where the pages are silent (causal alignment, GQA head mapping,
cache layout, slot formula, output dtype) are the conventions listed in the
module docstrings below.  Every function here is pinned by a CPU test against
something other than itself.
"""
from .bits import as_f64, bf16_bits_to_f64, f32_to_bf16_bits_rne  # noqa: F401
from .pool import RefBlockPool  # noqa: F401
from .scatter import ref_reshape_and_cache  # noqa: F401
from .attention import (  # noqa: F401
    causal_attention,
    gather_sequence,
    ref_attention_dense,
    ref_attention_paged,
)
from .bruteforce import ref_bruteforce  # noqa: F401
