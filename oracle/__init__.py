"""fp64 CPU oracle for exact attention. Test infrastructure only (see oracle.py)."""
from .oracle import *  # noqa: F401,F403
from .oracle import (MASK_NONE, MASK_CAUSAL_TOP_LEFT, MASK_CAUSAL_BOTTOM_RIGHT,  # noqa: F401
                     token_metadata, allowed, explicit_mask, attention, attention_explicit,
                     attention_per_sequence, attention_bwd, attention_explicit_bwd,
                     lse_combine, attention_key_range, philox4x32_10,
                     dropout_threshold, dropout_keep)
