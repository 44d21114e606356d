"""Oracle package: TEST INFRASTRUCTURE ONLY.

Plain CPU references for the masked grouped-query attention forward pass and
the KV-cache append that feeds decode.  Only tests/, the smoke check and the
benchmark's CPU-baseline leg may import it.  Nothing here imports the HIP
library or its binding, and the library never imports this package.
"""
from .attention_fp64 import (  # noqa: F401
    apply_softcap,
    attention,
    attention_rows,
    band,
    band_row,
    visible,
    kv_head,
    probabilities,
    scale,
    softmax_masked,
    visible_pairs,
)
from .brute import attention_brute  # noqa: F401
from .kvcache import kv_cache_update  # noqa: F401
