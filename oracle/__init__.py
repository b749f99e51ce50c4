"""fp64 CPU oracle (test infrastructure only; see kata_oracle)."""
from .kata_oracle import (  # noqa: F401
    convex_gate,
    decode_state,
    decode_step,
    feature_dim,
    feature_map,
    feature_pairs,
    feature_weights,
    forward_chunked,
    forward_quadratic,
    forward_rows,
)
