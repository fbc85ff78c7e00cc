// Host-side launchers of the libpsa kernels. Arguments are validated by the
// C-ABI layer (psa_abi.cpp) before any of these is called; the launchers only
// pick a template instance and a grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace psa {

// PsaPackQkv: qkv [BH*4, KD, N] (the NCHW tensor viewed per head) -> packed [4, BH, N, KD].
hipError_t launch_pack_qkv(const void* qkv, void* packed, int BH, int KD, int N, int elt_bytes,
                           hipStream_t stream);

// PsaMergeAttn (slot0 = 0, rows = o2 [2, BH, N, KD]) and PsaExtractV (slot0 = 2,
// rows = packed [4, BH, N, KD]): rows[slot0 + j][bh] -> nchw [BH*2, KD, N].
hipError_t launch_rows_to_nchw(const void* rows, void* nchw, int BH, int KD, int N, int slot0,
                               int elt_bytes, hipStream_t stream);

// FA2 forward on [BH, n, D] tensors. ws / ws_bytes: workspace for the tail
// split (used only if it holds fa2_fwd_split_bytes; may be null).
hipError_t launch_fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                          int n_q, int n_k, int D, float scale, bool bf16, void* ws,
                          size_t ws_bytes, hipStream_t stream);
size_t fa2_fwd_split_bytes(int BH, int n_q, int n_k, int D, bool bf16);

// Fused PSA forward: qkv [B, 4hKD, H, W] -> out [B, 2hKD, H, W] (+ V residual, + LSE).
hipError_t launch_psa_fused_fwd(const void* qkv, void* out, void* vres, float* lse, int BH, int KD,
                                int N, float scale, bool bf16, void* ws, size_t ws_bytes,
                                hipStream_t stream);
size_t psa_fused_split_bytes(int BH, int KD, int N, bool bf16);

// PSA backward (bf16): qkv, out, dout [, dvres] NCHW + lse -> dqkv NCHW.
// workspace: 2 * BH * N floats (-Delta, LSE * log2(e)).
hipError_t launch_psa_fused_bwd(const void* qkv, const void* out, const float* lse, const void* dout,
                                const void* dvres, void* dqkv, float* workspace, int BH, int KD,
                                int N, float scale, bool bf16, hipStream_t stream);

// FA2 backward: -Delta and LSE * log2(e) into the workspace (2 * BH * n_q
// floats), then the dK/dV and dQ kernels.
hipError_t launch_fa2_bwd(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* workspace, int BH, int n_q, int n_k, int D, float scale, bool bf16,
                          hipStream_t stream);

// fa2_bwd with -Delta in the library's own device scratch (no allocation, no
// workspace argument): at most kNoAllocScratchBytes / 8 rows (BH * n_q).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;

// Set-up of the current device, which every entry point runs before its
// launches: the first call on a device looks up the device address of
// fa2_bwd_noalloc's scratch array (later calls return at once). Calls that
// arrive while it runs wait for it, so that the lookup never overlaps a
// launch of this library's kernels on another thread (HIP's symbol lookup
// has aborted the process when it did).
hipError_t init_device();
hipError_t launch_fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                  int BH, int n_q, int n_k, int D, float scale, bool bf16,
                                  hipStream_t stream);

// Detect-decode: boxes [B, 4, A] LTRB (float32 or bf16) + anchor grid [A] x3 -> out [B, 4, A].
hipError_t launch_detect_decode(const void* boxes, const float* anchor_x, const float* anchor_y,
                                const float* strides, void* out, int B, int64_t A, bool bf16,
                                hipStream_t stream);

// CIoU loss on [4, N] float32 boxes: per-anchor loss, iou, v, alpha.
hipError_t launch_ciou_fwd(const float* pred, const float* target, float* loss, float* iou,
                           float* v, float* alpha, int64_t N, hipStream_t stream);

// CIoU backward: dpred [4, N] from the saved iou, v, alpha and dloss [N].
hipError_t launch_ciou_bwd(const float* pred, const float* target, const float* iou,
                           const float* v, const float* alpha, const float* dloss, float* dpred,
                           int64_t N, hipStream_t stream);

}  // namespace psa
