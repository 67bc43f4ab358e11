"""CPU oracle for the KDA recurrence (test infrastructure only; see kda_oracle)."""
from .kda_oracle import (  # noqa: F401
    compose,
    decode_step,
    prefill,
    recurrence,
    rel_l2,
    segment_fragments,
    transition,
    verify_block,
)
