"""Plain fp64 CPU oracle for one decoding step of Flash-dLLM's per-layer hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``kv_cache_attention_flash_amd``) never imports, calls or links it, and this
package imports nothing from the product path: the two share no code.

Sources (PUBLIC web pages about one preprint; cited by short key):

* [P4] "Flash-dLLM: I/O-Aware KV Caching and Parallel Decoding for Fast,
  Memory-Efficient Diffusion LLMs", summary page on ai4snews.wisdomeyes.cn,
  paragraphs 1-5 (P4 para 1: Flash-Cache fusion of QKV projection, rotary
  embedding and cache write; scheduled attention over a block table.
  P4 para 2: selective cache update, window plus tracking budget of most-attended
  tokens.  P4 para 3: Flash-Verify two-view mask and causal-order acceptance).
* [P2] the arXiv abstract page of the same preprint (abstract).

``reference`` holds one per-layer step; ``loop`` chains such steps into
a weight-free multi-step loop (planning rules stated in its docstring);
``lm_head`` is the mask-view confidence producer that feeds the accept scan.

Every function states the passage it follows.  Where the pages are silent the
function states the reading it takes; the same readings are listed in the
repository's design notes.

Pinned by ``tests/test_oracle_*.py`` against closed forms, invariants,
hand-worked examples in ``tests/golden/`` and brute force on tiny inputs.
"""

from .reference import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    qkv_projection,
    rope_rotate,
    physical_slots,
    flash_cache_step,
    visibility_mask,
    attention,
    attention_mass,
    top_b,
    accept_length,
    decode_step,
)
from .loop import (  # noqa: F401
    STAGE_UPDATE,
    STAGE_REFRESH,
    STAGE_DONE,
    plan_step,
    hidden_rows,
    decode_loop,
)
from .lm_head import (  # noqa: F401
    lm_head_confidence,
    verify_chain,
)
