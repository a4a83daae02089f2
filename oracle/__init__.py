"""fp64 CPU oracle (test infrastructure only; see attention.py and encoder_layer.py)."""
from .attention import (  # noqa: F401
    admitted_pairs, as_f64, attention_head, causal_rows, encoder_admit_mask, encoder_attention,
    key_interval, merge_partials, partial_attention, qkv_projection, softmax_probabilities,
    split_heads, verify_attention,
)
