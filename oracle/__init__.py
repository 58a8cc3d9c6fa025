"""Plain fp64 CPU oracle for E2D2's block-masked attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or load this
package: only the tests, the smoke check and the bench's CPU-baseline leg do.  It
shares no code with the HIP library (masked_attention_amd) and the two never import
each other; both take their inputs from the ``synth`` generator.

The method computes exact masked softmax attention, so every function here is that
definition written out: an explicit boolean mask, fp64 scores, one softmax per query
row over all allowed keys, O and LSE.  Pins that tie it to the pages (pair counts
from the FLOPs table, the block-size-1 and block-size-L reductions, exact caching,
brute force on tiny shapes) live in tests/test_oracle_pins.py.

Parity pinned: every function in this package is pinned by at least one test that
does not re-type its formula (see the module docstrings).
"""
from .masks import (  # noqa: F401
    block_of,
    encoder_mask,
    decoder_mask,
    denoise_mask,
    bd3lm_mask,
    count_pairs,
    count_tiles,
)
from .attention import (  # noqa: F401
    masked_softmax_attention,
    encoder_blockcausal,
    decoder_fused,
    train_fwd,
    denoise_step,
    bd3lm_layer,
    kv_cache_append,
)
from .backward import (  # noqa: F401
    masked_softmax_attention_grad,
    train_bwd,
)
from .layer import (  # noqa: F401
    round_bf16,
    decoder_layer_denoise,
)
