/*
 * psa.h - C ABI of libpsa.so, the MI355X (gfx950) PSA-block attention path.
 *
 * The path (vision-rs book, "Custom Kernels", section "Position-Sensitive
 * Attention (PSA)"): a QKV convolution's NCHW output [B, qkv_h, H, W], whose
 * channels come in per-head groups ordered Q, K, V_lo, V_hi (KEY_DIM apiece),
 * is repacked to [4, BH, N, KEY_DIM]; Flash Attention 2 runs once per V half
 * with HEAD_DIM = KEY_DIM, sharing Q and K; the two outputs are merged back to
 * NCHW [B, c, H, W]; the two V halves are also returned to NCHW, where the
 * block's residual branch uses them. psa_attention_fwd does all of it in one kernel.
 *
 * Notation: h = heads, KD = key_dim, N = H*W, BH = B*h, n = y*W + x,
 * bh = b*h + i (head i of batch item b), qkv_h = 4*h*KD, c = 2*h*KD.
 * Channel of slot s (0 Q, 1 K, 2 V_lo, 3 V_hi) of head i: i*4*KD + s*KD + d.
 * Channel of half j (0 lo, 1 hi) of head i in merged/extracted outputs:
 * i*2*KD + j*KD + d.
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers to contiguous row-major buffers, 16-byte
 *    aligned. The caller owns every buffer; the library allocates nothing and
 *    never synchronizes. Its only state is a thread-local error string and a
 *    per-process cache of device properties (CU count of each device, the
 *    occupancy of each kernel) that launches are sized with.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued asynchronously on it. The stream and every buffer belong
 *    to the calling thread's current HIP device (hipSetDevice): launch sizes
 *    and fa2_bwd_noalloc's scratch are taken for that device.
 *  - Outputs are overwritten, never accumulated into. Inputs are read only.
 *  - Every argument is validated before anything is launched. On any error
 *    nothing is enqueued, nothing is written, the status says which class of
 *    error it was and psa_last_error() names the entry point and the argument.
 *  - Element type: PSA_BF16 (bfloat16 storage, float32 accumulation and
 *    float32 softmax, results rounded to nearest even) or PSA_F32 (float32
 *    throughout). Layout entry points move bit patterns and never round.
 *  - KD / head_dim must be one of 16, 32, 64, 128 (FA2's HEAD_DIM is a
 *    compile-time power of two: vision-rs book, "Custom Kernels", section
 *    "Flash Attention 2").
 *  - Input and output byte ranges must not overlap (PSA_ERR_ALIAS).
 *  - No C++ exception crosses this interface.
 */
#ifndef PSA_H
#define PSA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PSA_ABI_VERSION 4

/* Element type. A C caller may pass any int; the library rejects values other
 * than these two with PSA_ERR_UNSUPPORTED. Compiled as C++, the enum gets int as
 * its fixed underlying type (the same size and ABI as the C enum), so that such
 * a value is a valid psa_dtype there too and the check on it stays meaningful. */
#ifdef __cplusplus
typedef enum psa_dtype : int {
#else
typedef enum psa_dtype {
#endif
  PSA_F32 = 0,
  PSA_BF16 = 1
} psa_dtype;

typedef enum psa_status {
  PSA_OK = 0,
  PSA_ERR_NULL = 1,        /* a required pointer is NULL */
  PSA_ERR_SHAPE = 2,       /* a dimension is <= 0 or a size overflows */
  PSA_ERR_UNSUPPORTED = 3, /* key_dim/head_dim/dtype/scale outside what is built */
  PSA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  PSA_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
  PSA_ERR_LAUNCH = 6       /* the HIP runtime rejected a launch */
} psa_status;

/*
 * PsaPackQkv (vision-rs book, "Custom Kernels", "Position-Sensitive Attention
 * (PSA)", PsaPackQkv):
 *   packed[s][b*h+i][n][d] = qkv[b][i*4*KD + s*KD + d][y][x]
 * qkv_nchw: [B, 4*h*KD, H, W] input.  packed: [4, B*h, H*W, KD] output.
 * A pure permutation of elements (bit copy).
 */
psa_status psa_pack_qkv(const void* qkv_nchw, void* packed, int B, int heads, int key_dim,
                        int H, int W, psa_dtype dtype, void* stream);

/*
 * PsaExtractV (same page and section, PsaExtractV bullet: both V channel
 * groups returned to NCHW, where the block's residual branch reads them):
 *   v_nchw[b][i*2*KD + j*KD + d][y][x] = packed[2+j][b*h+i][n][d]
 * packed: [4, B*h, H*W, KD] input (only slots 2 and 3 are read).
 * v_nchw: [B, 2*h*KD, H, W] output. Bit copy.
 */
psa_status psa_extract_v(const void* packed, void* v_nchw, int B, int heads, int key_dim,
                         int H, int W, psa_dtype dtype, void* stream);

/*
 * PsaMergeAttn (same page and section, PsaMergeAttn bullet: the two FA2
 * outputs returned to the NCHW layout [B, c, H, W]):
 *   out_nchw[b][i*2*KD + j*KD + d][y][x] = o2[j][b*h+i][n][d]
 * o2: [2, B*h, H*W, KD] input (half 0 = attention over V_lo, 1 = over V_hi).
 * out_nchw: [B, 2*h*KD, H, W] output. Bit copy.
 */
psa_status psa_merge_attn(const void* o2, void* out_nchw, int B, int heads, int key_dim,
                          int H, int W, psa_dtype dtype, void* stream);

/*
 * Forward workspaces (fa2_fwd, psa_attention_fwd). A bf16 forward launch
 * gives each workgroup one tile of queries. When the tiles fill the device's
 * resident workgroup slots a whole number of times plus a short last round,
 * that round would run on a few CUs while the rest idle; with a workspace the
 * launch instead cuts the last round's tiles into key-range pieces, spreads
 * them over the whole device and merges them with the log-sum-exp weights of
 * the online softmax (a second, small kernel on the same stream). The
 * *_workspace_bytes functions give the bytes this needs on the CURRENT device
 * (0: these sizes do not split; also 0 for PSA_F32 and for invalid sizes).
 * workspace may be NULL, or smaller than that: the launch then runs unsplit,
 * with the same results to within rounding. A workspace must be 16-byte
 * aligned and must not overlap any other argument; its contents on entry do
 * not matter and on return are unspecified. Two launches in flight at once
 * must not share one.
 */
size_t fa2_fwd_workspace_bytes(int BH, int n_q, int n_k, int head_dim, psa_dtype dtype);

/*
 * Flash Attention 2 forward (vision-rs book, "Custom Kernels", "Flash
 * Attention 2": online softmax over [BATCH*N_HEADS, N_CTX, HEAD_DIM] tensors;
 * the n_q x n_k score matrix is never stored):
 *   o[bh][n][:] = sum_m softmax_m(scale * q[bh][n] . k[bh][m]) * v[bh][m][:]
 *   lse[bh][n]  = ln sum_m exp(scale * q[bh][n] . k[bh][m])      (natural log)
 * q: [BH, n_q, head_dim]; k, v: [BH, n_k, head_dim]; o: [BH, n_q, head_dim];
 * lse: [BH, n_q] float32, or NULL to skip it. No mask, no dropout, no bias.
 * scale must be finite and > 0. workspace / workspace_bytes: see "Forward
 * workspaces" above (NULL allowed).
 */
psa_status fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int BH, int n_q, int n_k, int head_dim, float scale, psa_dtype dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Flash Attention 2 backward: the dQ kernel and the dK/dV kernel are separate
 * launches with their own grids (vision-rs book, "Custom Kernels", "Flash
 * Attention 2"). With P = exp(scale*q k^T - lse), Delta = rowsum(dout * o),
 * dS = P * (dout v^T - Delta):
 *   dq = scale * dS k,  dk = scale * dS^T q,  dv = P^T dout.
 * q, o, dout, dq: [BH, n_q, head_dim]; k, v, dk, dv: [BH, n_k, head_dim];
 * lse: [BH, n_q] float32 as written by fa2_fwd; workspace: caller-owned
 * float32 scratch of fa2_bwd_workspace_bytes(BH, n_q) bytes (the library keeps
 * -Delta and LSE * log2(e) there between its launches; its contents on return
 * are not part of the results).
 * scale must be the one given to fa2_fwd.
 */
psa_status fa2_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, float* workspace,
                   int BH, int n_q, int n_k, int head_dim, float scale, psa_dtype dtype,
                   void* stream);

/* Bytes of workspace fa2_bwd needs: 2 * BH * n_q floats. 0 if a size is invalid. */
size_t fa2_bwd_workspace_bytes(int BH, int n_q);

/*
 * fa2_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc):
 * the same computation, results bit-identical to fa2_bwd's, with no workspace
 * argument. The -Delta and LSE * log2(e) rows live instead in a scratch array of
 * PSA_NOALLOC_SCRATCH_BYTES that the library's code object holds in device
 * memory; each GPU it runs on has its own copy, held until the process ends.
 * Its device address is looked up once per GPU, by the first call of any
 * entry point on that GPU, before that call launches anything. The entry
 * point calls no allocating routine. Limit: BH * n_q <=
 * PSA_NOALLOC_SCRATCH_BYTES / 8 (2,097,152 rows); larger calls return
 * PSA_ERR_SHAPE before anything is launched (use fa2_bwd with a workspace).
 * Every call on one GPU shares that scratch: calls whose executions overlap
 * on one GPU (on different streams, or from several host threads without
 * ordering) race and give wrong results; calls ordered on one stream do not.
 * Other arguments, layouts and errors as fa2_bwd.
 */
#define PSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
psa_status fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int BH, int n_q, int n_k, int head_dim, float scale, psa_dtype dtype,
                           void* stream);

/*
 * The whole PSA forward in one kernel: PsaPackQkv, FA2 over (Q, K, V_lo) and
 * (Q, K, V_hi) and PsaMergeAttn (vision-rs book, "Custom Kernels",
 * "Position-Sensitive Attention (PSA)"), fused as teenygrad's book says custom
 * ops must be ("Your Kernel as a Graph Op", "Where fusion happens"). One
 * softmax serves both halves, since they share Q and K:
 *   out_nchw[b][i*2*KD + j*KD + d][y][x] = FA2(Q, K, V_j)[b*h+i][n][d]
 * qkv_nchw: [B, 4*h*KD, H, W]; out_nchw: [B, 2*h*KD, H, W].
 * v_nchw: [B, 2*h*KD, H, W] V residual exactly as psa_extract_v writes it, or
 * NULL to skip it. lse: [B*h, H*W] float32, or NULL.
 * scale must be finite and > 0 (the PSA block uses key_dim ** -0.5).
 * workspace / workspace_bytes: see "Forward workspaces" above (NULL allowed).
 */
psa_status psa_attention_fwd(const void* qkv_nchw, void* out_nchw, void* v_nchw, float* lse,
                             int B, int heads, int key_dim, int H, int W, float scale,
                             psa_dtype dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Workspace bytes for psa_attention_fwd; see "Forward workspaces" above. */
size_t psa_attention_fwd_workspace_bytes(int B, int heads, int key_dim, int H, int W,
                                         psa_dtype dtype);

/*
 * PSA backward: the gradient of psa_attention_fwd's outputs with respect to
 * qkv_nchw, i.e. the forward's steps (PsaPackQkv, FA2 over (Q, K, V_lo) and
 * (Q, K, V_hi), PsaMergeAttn, PsaExtractV; vision-rs book, "Custom Kernels",
 * "Position-Sensitive Attention (PSA)" and "Flash Attention 2") taken in
 * reverse. With P = exp(scale*Q K^T - lse), dO = the two halves of dout_nchw,
 * O = the two halves of out_nchw, V = [V_lo | V_hi], Delta = rowsum(dO * O):
 *   dS = P * (dO V^T - Delta)
 *   dqkv[Q]  = scale * dS K        (the sum of both halves' dQ)
 *   dqkv[K]  = scale * dS^T Q      (the sum of both halves' dK)
 *   dqkv[V]  = P^T dO + dv_nchw    (per half; the V residual's gradient adds)
 * written in the NCHW channel order of qkv_nchw. No gradient flows through lse.
 * qkv_nchw: [B, 4*h*KD, H, W] forward input. out_nchw, lse: the forward's
 * output [B, 2*h*KD, H, W] and LSE [B*h, H*W] (as psa_attention_fwd wrote them).
 * dout_nchw: [B, 2*h*KD, H, W] gradient of out. dv_nchw: [B, 2*h*KD, H, W]
 * gradient of the V residual, or NULL for none. dqkv_nchw: [B, 4*h*KD, H, W]
 * output. workspace: caller-owned float32 scratch of
 * psa_attention_bwd_workspace_bytes(B, heads, H, W) bytes. PSA_BF16 (matrix
 * cores, one backward for both halves) or PSA_F32 (float32 on the VALU, one V
 * half after the other). scale: the forward's.
 */
psa_status psa_attention_bwd(const void* qkv_nchw, const void* out_nchw, const float* lse,
                             const void* dout_nchw, const void* dv_nchw, void* dqkv_nchw,
                             float* workspace, int B, int heads, int key_dim, int H, int W,
                             float scale, psa_dtype dtype, void* stream);

/* Bytes of workspace psa_attention_bwd needs: 2 * B*h * H*W floats. 0 if a size is invalid. */
size_t psa_attention_bwd_workspace_bytes(int B, int heads, int H, int W);

/*
 * Detect-decode (vision-rs book, "Custom Kernels", section "Detect-decode";
 * teenygrad book, "Your Kernel as a Graph Op", section "A real one"): raw LTRB
 * box distances plus a precomputed anchor grid to [cx, cy, w, h] boxes in one
 * pass. For batch item b and anchor a, with (l, t, r, bt) = boxes[b][0..3][a]
 * and (ax, ay, s) = (anchor_x[a], anchor_y[a], strides[a]):
 *   x1 = ax - l, y1 = ay - t, x2 = ax + r, y2 = ay + bt
 *   out[b][0..3][a] = ((x1 + x2)/2 * s, (y1 + y2)/2 * s, (x2 - x1) * s, (y2 - y1) * s)
 * boxes: [B, 4, A] in dtype (PSA_F32 or PSA_BF16). out: [B, 4, A], same dtype
 * (the op keeps the input's shape and type). anchor_x, anchor_y, strides: [A]
 * float32 each, the anchor centres in grid units and the grid's stride in
 * pixels. Arithmetic is float32; a bf16 result is rounded once, to nearest
 * even. B <= 65535, A < 2^31 - 256. out must not overlap any input.
 */
psa_status detect_decode(const void* boxes, const float* anchor_x, const float* anchor_y,
                         const float* strides, void* out, int B, long long A, psa_dtype dtype,
                         void* stream);

/*
 * CIoU loss forward (vision-rs book, "Custom Kernels", section "Loss kernels",
 * ciou): per anchor n, the complete-IoU loss of box pred[.][n] against
 * target[.][n] (rows cx, cy, w, h) plus the iou, v and alpha its backward
 * reuses:
 *   IoU = I / (w h + w_t h_t - I + eps), I the overlap area
 *   v = 4/pi^2 (atan(w_t / (h_t + eps)) - atan(w / (h + eps)))^2
 *   alpha = v / (v - IoU + 1 + eps)
 *   loss = 1 - IoU + rho^2 / (c^2 + eps) + alpha v
 * with rho the distance of the centres, c the diagonal of the smallest box
 * enclosing both, eps = 1e-7. pred, target: [4, N] float32. loss, iou, v,
 * alpha: [N] float32 outputs. Arithmetic is float32. N < 2^31 - 256.
 */
psa_status ciou_loss_fwd(const float* pred, const float* target, float* loss, float* iou,
                         float* v, float* alpha, long long N, void* stream);

/*
 * CIoU loss backward (same section): dpred[k][n] = dloss[n] * d loss[n] /
 * d pred[k][n], alpha held constant (no gradient flows through it; targets
 * get none). iou, v, alpha: the [N] values ciou_loss_fwd saved for the same
 * pred and target. dloss: [N] float32. dpred: [4, N] float32 output.
 */
psa_status ciou_loss_bwd(const float* pred, const float* target, const float* iou,
                         const float* v, const float* alpha, const float* dloss, float* dpred,
                         long long N, void* stream);

/* Message of the last error on this thread ("" after a success). */
const char* psa_last_error(void);

/* PSA_ABI_VERSION of the loaded library. */
int psa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PSA_H */
