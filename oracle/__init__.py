"""CPU oracle -- test infrastructure only (tests, smoke check, CPU baseline)."""
from .compressed_linear_oracle import (  # noqa: F401
    TOL_REL,
    activations,
    round_to_act,
    dense_plane,
    sparse_plane,
    lowrank_factors,
    reconstruct,
    forward,
    bound,
    forward_and_bound,
    debug_planes,
)
