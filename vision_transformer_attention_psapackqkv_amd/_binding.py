"""ctypes binding of libpsa.so (the C ABI declared in include/psa.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch supplies device memory (``torch.empty`` for outputs) and the
current stream. There is no fallback of any kind: if the library is missing or
a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpsa.so")

PSA_F32, PSA_BF16 = 0, 1
STATUS_NAMES = {0: "PSA_OK", 1: "PSA_ERR_NULL", 2: "PSA_ERR_SHAPE", 3: "PSA_ERR_UNSUPPORTED",
                4: "PSA_ERR_ALIGN", 5: "PSA_ERR_ALIAS", 6: "PSA_ERR_LAUNCH"}

# Every exported symbol with its ctypes signature (same order and types as include/psa.h).
_P, _I, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "psa_pack_qkv": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "psa_extract_v": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "psa_merge_attn": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fa2_fwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "fa2_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, ctypes.c_size_t, _P]),
    "fa2_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa2_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
    "fa2_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "psa_attention_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, ctypes.c_size_t, _P]),
    "psa_attention_fwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I]),
    "psa_attention_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "psa_attention_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "detect_decode": (_I, [_P, _P, _P, _P, _P, _I, ctypes.c_longlong, _I, _P]),
    "ciou_loss_fwd": (_I, [_P, _P, _P, _P, _P, _P, ctypes.c_longlong, _P]),
    "ciou_loss_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_longlong, _P]),
    "psa_last_error": (ctypes.c_char_p, []),
    "psa_abi_version": (_I, []),
}


class PsaError(RuntimeError):
    """A libpsa entry point returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library() -> ctypes.CDLL:
    """Loads libpsa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpsa.so not found at {LIB_PATH}: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise PsaError(status, load_library().psa_last_error().decode())


def _on_device(fn):
    """Runs a binding entry point with its first tensor argument's GPU as the current HIP
    device: the library sizes launches (and picks fa2_bwd_noalloc's scratch) for the current
    device, and the tensors and stream passed are that GPU's."""
    @functools.wraps(fn)
    def wrapper(t, *args, **kwargs):
        if isinstance(t, torch.Tensor) and t.device.type == "cuda" and t.device.index != torch.cuda.current_device():
            with torch.cuda.device(t.device):
                return fn(t, *args, **kwargs)
        return fn(t, *args, **kwargs)
    return wrapper


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PSA_BF16
    if t.dtype == torch.float32:
        return PSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _arg(t, name: str, shape=None, dtype=None, like: torch.Tensor | None = None, min_bytes=None):
    """Checks a tensor handed to the C ABI against the sizes the call will use: its shape and
    dtype (where given), at least ``min_bytes`` bytes (a workspace), a GPU tensor on ``like``'s
    device, contiguous. Raises ValueError before anything is allocated or launched: the kernels
    trust these sizes, so a wrong one would read or write past the tensor."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {min_bytes}")
    _dev(t, name)
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")
    return t


def _float_dtype(t: torch.Tensor, name: str):
    if t.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"{name} has dtype {t.dtype}: use torch.bfloat16 or torch.float32")
    return t.dtype


def _nchw(qkv, heads, key_dim, name="qkv"):
    """(B, H, W) of an NCHW qkv tensor ``[B, 4*heads*key_dim, H, W]``."""
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 4:
        raise ValueError(f"{name} must be a 4-D NCHW tensor")
    B, C, H, W = qkv.shape
    if C != 4 * heads * key_dim:
        raise ValueError(f"{name} has {C} channels, expected 4*heads*key_dim = {4 * heads * key_dim}")
    _float_dtype(qkv, name)
    return B, H, W


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def default_scale(key_dim: int) -> float:
    return float(key_dim) ** -0.5


@_on_device
def psa_pack_qkv(qkv: torch.Tensor, heads: int, key_dim: int, out: torch.Tensor | None = None):
    """qkv NCHW ``[B, 4*heads*key_dim, H, W]`` -> packed ``[4, B*heads, H*W, key_dim]``."""
    B, H, W = _nchw(qkv, heads, key_dim)
    _arg(qkv, "qkv")
    shape = (4, B * heads, H * W, key_dim)
    if out is None:
        out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device)
    _arg(out, "out", shape, qkv.dtype, like=qkv)
    _check(load_library().psa_pack_qkv(qkv.data_ptr(), out.data_ptr(), B, heads,
                                       key_dim, H, W, _dtype_code(qkv), _stream(qkv)))
    return out


def _rows_to_nchw(fn_name, rows, slots, B, heads, key_dim, H, W, out):
    _arg(rows, "input", (slots, B * heads, H * W, key_dim))
    _float_dtype(rows, "input")
    shape = (B, 2 * heads * key_dim, H, W)
    if out is None:
        out = torch.empty(shape, dtype=rows.dtype, device=rows.device)
    _arg(out, "out", shape, rows.dtype, like=rows)
    fn = getattr(load_library(), fn_name)
    _check(fn(rows.data_ptr(), out.data_ptr(), B, heads, key_dim, H, W,
              _dtype_code(rows), _stream(rows)))
    return out


@_on_device
def psa_extract_v(packed, B, heads, key_dim, H, W, out=None):
    """packed ``[4, B*heads, H*W, key_dim]`` -> V residual NCHW ``[B, 2*heads*key_dim, H, W]``."""
    return _rows_to_nchw("psa_extract_v", packed, 4, B, heads, key_dim, H, W, out)


@_on_device
def psa_merge_attn(o2, B, heads, key_dim, H, W, out=None):
    """o2 ``[2, B*heads, H*W, key_dim]`` -> NCHW ``[B, 2*heads*key_dim, H, W]``."""
    return _rows_to_nchw("psa_merge_attn", o2, 2, B, heads, key_dim, H, W, out)


def _workspace(ws, nbytes, like):
    """(pointer, bytes) of a forward workspace: a new one of ``nbytes`` if ``ws`` is None,
    else the given tensor, of any size (a smaller or empty one runs the launch unsplit)."""
    if ws is None:
        if nbytes == 0:
            return None, 0
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=like.device)
    _arg(ws, "workspace", like=like)
    return (ws.data_ptr() if ws.numel() else None), ws.numel() * ws.element_size()


def fa2_fwd_workspace_bytes(BH, n_q, n_k, head_dim, dtype=torch.bfloat16):
    """Workspace bytes that let fa2_fwd split the last round of its grid (0: no split)."""
    code = PSA_BF16 if dtype == torch.bfloat16 else PSA_F32
    return load_library().fa2_fwd_workspace_bytes(BH, n_q, n_k, head_dim, code)


def psa_attention_fwd_workspace_bytes(B, heads, key_dim, H, W, dtype=torch.bfloat16):
    """Workspace bytes that let psa_attention_fwd split the last round of its grid (0: no split)."""
    code = PSA_BF16 if dtype == torch.bfloat16 else PSA_F32
    return load_library().psa_attention_fwd_workspace_bytes(B, heads, key_dim, H, W, code)


def _qkv3(q, k, v):
    """(BH, n_q, D, n_k) of FA2's ``[BH, n, D]`` q, k, v (k and v share q's BH, D and dtype)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D [BH, n_q, D] tensor")
    _float_dtype(q, "q")
    _arg(q, "q")
    BH, n_q, D = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 3:
        raise ValueError("k must be a 3-D [BH, n_k, D] tensor")
    n_k = k.shape[1]
    _arg(k, "k", (BH, n_k, D), q.dtype, like=q)
    _arg(v, "v", (BH, n_k, D), q.dtype, like=q)
    return BH, n_q, D, n_k


@_on_device
def fa2_fwd(q, k, v, scale=None, out=None, lse=None, want_lse=True, workspace=None):
    """FA2 forward on ``[BH, n, D]`` tensors; returns ``(o, lse)`` (lse is None if not wanted).

    ``workspace``: None allocates the bytes ``fa2_fwd_workspace_bytes`` asks for; a given
    GPU tensor is used as is (an empty one runs the launch without the tail split)."""
    BH, n_q, D, n_k = _qkv3(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _arg(out, "out", q.shape, q.dtype, like=q)
    if lse is None and want_lse:
        lse = torch.empty((BH, n_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _arg(lse, "lse", (BH, n_q), torch.float32, like=q)
    s = default_scale(D) if scale is None else float(scale)
    lib = load_library()
    code = _dtype_code(q)
    wp, wb = _workspace(workspace, lib.fa2_fwd_workspace_bytes(BH, n_q, n_k, D, code), q)
    _check(lib.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       _ptr(lse), BH, n_q, n_k, D, s, code, wp, wb, _stream(q)))
    return out, lse


@_on_device
def fa2_bwd(q, k, v, o, dout, lse, scale=None, workspace=None):
    """FA2 backward; returns ``(dq, dk, dv)``.

    ``workspace``: a GPU tensor of at least ``fa2_bwd_workspace_bytes(BH, n_q)`` bytes
    (2 * BH * n_q floats), or None to allocate one."""
    BH, n_q, D, n_k = _qkv3(q, k, v)
    _arg(o, "o", q.shape, q.dtype, like=q)
    _arg(dout, "dout", q.shape, q.dtype, like=q)
    _arg(lse, "lse", (BH, n_q), torch.float32, like=q)
    lib = load_library()
    nbytes = lib.fa2_bwd_workspace_bytes(BH, n_q)
    if workspace is not None:
        _arg(workspace, "workspace", min_bytes=nbytes, like=q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=q.device)
    s = default_scale(D) if scale is None else float(scale)
    _check(lib.fa2_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       workspace.data_ptr(), BH, n_q, n_k, D, s, _dtype_code(q), _stream(q)))
    return dq, dk, dv


NOALLOC_SCRATCH_BYTES = 16 << 20   # PSA_NOALLOC_SCRATCH_BYTES of include/psa.h


@_on_device
def fa2_bwd_noalloc(q, k, v, o, dout, lse, scale=None, dq=None, dk=None, dv=None):
    """FA2 backward through ``fa2_bwd_noalloc``: no workspace, the library keeps -Delta in its
    own device scratch (BH * n_q <= NOALLOC_SCRATCH_BYTES / 8). Returns ``(dq, dk, dv)``; pass
    them in to have nothing allocated at all. Calls that overlap on one GPU share that scratch
    and race; calls ordered on one stream do not."""
    BH, n_q, D, n_k = _qkv3(q, k, v)
    _arg(o, "o", q.shape, q.dtype, like=q)
    _arg(dout, "dout", q.shape, q.dtype, like=q)
    _arg(lse, "lse", (BH, n_q), torch.float32, like=q)
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        if t is not None:
            _arg(t, n, ref.shape, ref.dtype, like=q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    s = default_scale(D) if scale is None else float(scale)
    _check(load_library().fa2_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                          dv.data_ptr(), BH, n_q, n_k, D, s, _dtype_code(q), _stream(q)))
    return dq, dk, dv


@_on_device
def psa_attention_fwd(qkv, heads, key_dim, scale=None, want_v=True, want_lse=True,
                      out=None, v_out=None, lse=None, workspace=None):
    """Fused PSA forward on NCHW ``qkv``; returns ``(out, v_residual, lse)`` (None where not wanted).

    ``workspace`` as for :func:`fa2_fwd` (bytes from ``psa_attention_fwd_workspace_bytes``)."""
    B, H, W = _nchw(qkv, heads, key_dim)
    _arg(qkv, "qkv")
    shape = (B, 2 * heads * key_dim, H, W)
    if out is None:
        out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device)
    _arg(out, "out", shape, qkv.dtype, like=qkv)
    if v_out is None and want_v:
        v_out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device)
    if v_out is not None:
        _arg(v_out, "v_out", shape, qkv.dtype, like=qkv)
    if lse is None and want_lse:
        lse = torch.empty((B * heads, H * W), dtype=torch.float32, device=qkv.device)
    if lse is not None:
        _arg(lse, "lse", (B * heads, H * W), torch.float32, like=qkv)
    s = default_scale(key_dim) if scale is None else float(scale)
    lib = load_library()
    code = _dtype_code(qkv)
    wp, wb = _workspace(workspace, lib.psa_attention_fwd_workspace_bytes(B, heads, key_dim, H, W, code),
                        qkv)
    _check(lib.psa_attention_fwd(qkv.data_ptr(), out.data_ptr(), _ptr(v_out),
                                 _ptr(lse), B, heads, key_dim, H, W, s, code, wp, wb, _stream(qkv)))
    return out, v_out, lse


@_on_device
def psa_attention_bwd(qkv, out, lse, dout, heads, key_dim, dv=None, scale=None, dqkv=None,
                      workspace=None):
    """PSA backward: the gradient of ``psa_attention_fwd``'s outputs with respect to ``qkv``.

    ``out`` and ``lse`` are the forward's, ``dout`` the gradient of ``out``, ``dv`` the gradient
    of the V residual (None: none). Returns ``dqkv`` NCHW ``[B, 4*heads*key_dim, H, W]``.
    ``workspace``: a GPU tensor of at least ``psa_attention_bwd_workspace_bytes`` bytes, or None."""
    B, H, W = _nchw(qkv, heads, key_dim)
    _arg(qkv, "qkv")
    shape = (B, 2 * heads * key_dim, H, W)
    _arg(out, "out", shape, qkv.dtype, like=qkv)
    _arg(lse, "lse", (B * heads, H * W), torch.float32, like=qkv)
    _arg(dout, "dout", shape, qkv.dtype, like=qkv)
    if dv is not None:
        _arg(dv, "dv", shape, qkv.dtype, like=qkv)
    if dqkv is not None:
        _arg(dqkv, "dqkv", qkv.shape, qkv.dtype, like=qkv)
    lib = load_library()
    nbytes = lib.psa_attention_bwd_workspace_bytes(B, heads, H, W)
    if workspace is not None:
        _arg(workspace, "workspace", min_bytes=nbytes, like=qkv)
    if dqkv is None:
        dqkv = torch.empty_like(qkv)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=qkv.device)
    s = default_scale(key_dim) if scale is None else float(scale)
    _check(lib.psa_attention_bwd(qkv.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                 _ptr(dv), dqkv.data_ptr(), workspace.data_ptr(),
                                 B, heads, key_dim, H, W, s, _dtype_code(qkv), _stream(qkv)))
    return dqkv


class _PsaAttention(torch.autograd.Function):
    """Autograd node over the fused PSA forward and its backward (both in libpsa)."""

    @staticmethod
    def forward(ctx, qkv, heads, key_dim, scale, workspace):
        out, v_res, lse = psa_attention_fwd(qkv, heads, key_dim, scale=scale, workspace=workspace)
        ctx.save_for_backward(qkv, out, lse)
        ctx.heads, ctx.key_dim, ctx.scale = heads, key_dim, scale
        return out, v_res

    @staticmethod
    def backward(ctx, dout, dv_res):
        qkv, out, lse = ctx.saved_tensors
        if dout is None:
            dout = torch.zeros_like(out)
        dqkv = psa_attention_bwd(qkv, out, lse, dout.contiguous(), ctx.heads, ctx.key_dim,
                                 dv=None if dv_res is None else dv_res.contiguous(), scale=ctx.scale)
        return dqkv, None, None, None, None


def psa_attention(qkv, heads, key_dim, scale=None, workspace=None):
    """The PSA attention block as a differentiable op: NCHW ``qkv`` -> ``(out, v_residual)``.

    Forward is ``psa_attention_fwd``; the gradient with respect to ``qkv`` (from both outputs)
    is ``psa_attention_bwd``; bf16 or float32."""
    return _PsaAttention.apply(qkv, heads, key_dim, scale, workspace)


def _f32(t, name, shape=None):
    _dev(t, name)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


@_on_device
def detect_decode(boxes, anchor_x, anchor_y, strides, out=None):
    """LTRB ``boxes [B, 4, A]`` (float32 or bf16) + anchor grid ``[A]`` x3 (float32) ->
    ``[B, 4, A]`` cx, cy, w, h in the dtype of ``boxes``."""
    _dev(boxes, "boxes")
    if boxes.dim() != 3 or boxes.shape[1] != 4:
        raise ValueError(f"boxes must be [B, 4, A], got {tuple(boxes.shape)}")
    B, _, A = boxes.shape
    for t, n in ((anchor_x, "anchor_x"), (anchor_y, "anchor_y"), (strides, "strides")):
        _f32(t, n, (A,))
    if out is None:
        out = torch.empty_like(boxes)
    elif out.dtype != boxes.dtype or tuple(out.shape) != tuple(boxes.shape):
        raise ValueError("out must match boxes in shape and dtype")
    _check(load_library().detect_decode(boxes.data_ptr(), anchor_x.data_ptr(), anchor_y.data_ptr(),
                                        strides.data_ptr(), _dev(out, "out").data_ptr(), B, A,
                                        _dtype_code(boxes), _stream(boxes)))
    return out


@_on_device
def ciou_loss_fwd(pred, target, out=None):
    """``pred, target [4, N]`` float32 cx, cy, w, h -> ``(loss, iou, v, alpha)``, each ``[N]``
    (written into ``out``, a tuple of four such tensors, if given)."""
    _f32(pred, "pred")
    if pred.dim() != 2 or pred.shape[0] != 4:
        raise ValueError(f"pred must be [4, N], got {tuple(pred.shape)}")
    N = pred.shape[1]
    _f32(target, "target", (4, N))
    if out is None:
        out = tuple(torch.empty(N, dtype=torch.float32, device=pred.device) for _ in range(4))
    loss, iou, v, alpha = (_f32(t, n, (N,)) for t, n in zip(out, ("loss", "iou", "v", "alpha")))
    _check(load_library().ciou_loss_fwd(pred.data_ptr(), target.data_ptr(), loss.data_ptr(),
                                        iou.data_ptr(), v.data_ptr(), alpha.data_ptr(), N,
                                        _stream(pred)))
    return loss, iou, v, alpha


@_on_device
def ciou_loss_bwd(pred, target, iou, v, alpha, dloss, dpred=None):
    """Gradient ``[4, N]`` of ``sum(dloss * loss)`` w.r.t. ``pred`` from the forward's saved
    ``iou, v, alpha`` (alpha held constant)."""
    _f32(pred, "pred")
    if pred.dim() != 2 or pred.shape[0] != 4:
        raise ValueError(f"pred must be [4, N], got {tuple(pred.shape)}")
    N = pred.shape[1]
    _f32(target, "target", (4, N))
    for t, n in ((iou, "iou"), (v, "v"), (alpha, "alpha"), (dloss, "dloss")):
        _f32(t, n, (N,))
    if dpred is None:
        dpred = torch.empty((4, N), dtype=torch.float32, device=pred.device)
    _f32(dpred, "dpred", (4, N))
    _check(load_library().ciou_loss_bwd(pred.data_ptr(), target.data_ptr(), iou.data_ptr(),
                                        v.data_ptr(), alpha.data_ptr(), dloss.data_ptr(),
                                        dpred.data_ptr(), N, _stream(pred)))
    return dpred


def psa_abi_version() -> int:
    return load_library().psa_abi_version()
