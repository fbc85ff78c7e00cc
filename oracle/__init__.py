"""CPU oracle for the PSA attention path (psa_oracle) and the detect-decode / CIoU-loss kernels
(yolo_oracle). Test infrastructure only."""
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
from .yolo_oracle import ciou_backward, ciou_forward, detect_decode  # noqa: F401,E402
