"""CPU oracle (test infrastructure only; see oracle/mla.py)."""
from .mla import (  # noqa: F401
    absorbed_decode, attend, decode_output, fold_output_weights, folded_decode_output, output_projection, attention_score_macs, decode, gather_rows, latent_rows,
    mha_cache_values_per_token, mla_cache_values_per_token, prefill, query_projection,
    rope, rope_angles, round_to, widen,
)
