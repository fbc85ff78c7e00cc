"""CPU oracle for the PSA attention path (test infrastructure only; see psa_oracle)."""
from .psa_oracle import (  # noqa: F401
    attention,
    attention_bwd,
    default_scale,
    extract_v,
    merge_attn,
    pack_qkv,
    psa_backward,
    psa_forward,
    split_attn,
    unpack_qkv,
)
