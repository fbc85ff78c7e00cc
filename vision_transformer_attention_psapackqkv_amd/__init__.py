"""PSA-block attention on MI355X (gfx950): Python face of libpsa.so.

The library (HIP kernels + C ABI, include/psa.h) does all the work; this
package only marshals torch tensors into its entry points, which keep their C
names here.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    PSA_BF16,
    PSA_F32,
    PsaError,
    ciou_loss_bwd,
    ciou_loss_fwd,
    detect_decode,
    default_scale,
    fa2_bwd,
    fa2_bwd_noalloc,
    fa2_fwd,
    fa2_fwd_workspace_bytes,
    load_library,
    psa_abi_version,
    psa_attention,
    psa_attention_bwd,
    psa_attention_fwd,
    psa_attention_fwd_workspace_bytes,
    psa_extract_v,
    psa_merge_attn,
    psa_pack_qkv,
)
