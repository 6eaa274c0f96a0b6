"""CPU oracle for the Lookahead Sparse Attention (LSA) decode path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package.  The GPU
library never calls it, links it, or falls back to it.  It shares no code
with the GPU path and imports nothing from it.
"""

from .lsa_ref import (  # noqa: F401
    BLOCK,
    RefreshResult,
    attention,
    block_logits,
    compact,
    decode_step,
    decode_values,
    governing_refresh,
    kv_rows,
    level_logit,
    query_encoder,
    query_latent,
    round_bf16,
    refresh,
    seq_len_at,
    simulate,
    threshold,
    token_set,
    union,
    window_start,
)
from .denoise_ref import denoise_window, layer_softmax, top_p_set, vote  # noqa: F401,E402
