"""Plain CPU oracle for the PSA attention path (float64, numpy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library, and the HIP library never falls back to it.

What it follows (all citations are to the pages the method is described on):

* vision-rs book, "Custom Kernels", section "Position-Sensitive Attention
  (PSA)": PsaPackQkv reorders the NCHW output ``[B, qkv_h, H, W]`` of a QKV
  convolution, whose channels come in per-head groups ordered Q, K, V_lo,
  V_hi (KEY_DIM apiece), into ``[4, BH, N, KEY_DIM]``, the tensors FA2 takes; PsaExtractV returns the two V sections to NCHW, where the
  block's residual branch uses them; PsaMergeAttn writes the attention output back to NCHW
  ``[B, c, H, W]``. Flash Attention 2 runs once per V half with
  HEAD_DIM = KEY_DIM, sharing Q and K.
* same page, section "Flash Attention 2": standard FA2 over
  ``[BATCH*N_HEADS, N_CTX, HEAD_DIM]`` tensors. FA2's online softmax reaches,
  up to rounding, the plain definition softmax(scale * Q K^T) V, so this file
  writes that definition out with the full score row materialised. The
  backward is the textbook gradient of that definition (the page only names
  the dQ and dK/dV kernels).

Readings where the pages are silent (each is also listed in the design notes):
  * the softmax scale is KEY_DIM ** -0.5 unless given;
  * channel index inside a head group is ``sigma*KEY_DIM + d`` with
    sigma = 0 (Q), 1 (K), 2 (V_lo), 3 (V_hi), and heads are major:
    ``ch = i*4*KEY_DIM + sigma*KEY_DIM + d``;
  * spatial positions flatten as ``n = y*W + x`` and ``bh = b*heads + i``;
  * merge and extract write channel ``i*2*KEY_DIM + j*KEY_DIM + d`` for half
    j (0 = lo, 1 = hi) of head i;
  * attention is full (no mask, no dropout, no bias); LSE is the natural-log
    log-sum-exp of the scaled scores of a row.

All floating-point work is float64 on exact upcasts of the stored inputs.
The layout functions are pure permutations and work on any element dtype
(they are also used on raw bit patterns).
"""
from __future__ import annotations

import numpy as np


def default_scale(key_dim: int) -> float:
    """Softmax scale KEY_DIM ** -0.5 (reading: the usual 1/sqrt(d) of attention)."""
    return float(key_dim) ** -0.5


def _nchw_flat(b, ch, n, C: int, N: int):
    """Flat element offset of (b, ch, n=y*W+x) in a contiguous [B, C, H, W] tensor."""
    return (b * C + ch) * N + n


def pack_qkv(qkv: np.ndarray, B: int, heads: int, key_dim: int, H: int, W: int) -> np.ndarray:
    """PsaPackQkv: ``packed[s, b*heads+i, n, d] = qkv[b, i*4*KD + s*KD + d, y, x]``.

    vision-rs book, "Custom Kernels", "Position-Sensitive Attention (PSA)",
    PsaPackQkv bullet: NCHW ``[B, qkv_h, H, W]`` with per-head
    ``[Q | K | V_lo | V_hi]`` channel groups -> ``[4, BH, N, KEY_DIM]``.
    """
    KD, N, BH, C = key_dim, H * W, B * heads, 4 * heads * key_dim
    flat = np.asarray(qkv).reshape(-1)
    assert flat.size == B * C * N, "qkv has the wrong number of elements"
    bh, n, d = np.ix_(np.arange(BH), np.arange(N), np.arange(KD))
    b, i = bh // heads, bh % heads
    out = np.empty((4, BH, N, KD), dtype=flat.dtype)
    for s in range(4):
        ch = i * 4 * KD + s * KD + d
        out[s] = flat[_nchw_flat(b, ch, n, C, N)]
    return out


def extract_v(packed: np.ndarray, B: int, heads: int, key_dim: int, H: int, W: int) -> np.ndarray:
    """PsaExtractV: ``v[b, i*2*KD + j*KD + d, y, x] = packed[2+j, b*heads+i, n, d]``.

    vision-rs book, "Custom Kernels", "Position-Sensitive Attention (PSA)",
    PsaExtractV bullet: the V section of the packed tensor, back in NCHW.
    """
    KD, N, BH, C = key_dim, H * W, B * heads, 2 * heads * key_dim
    packed = np.asarray(packed).reshape(4, BH, N, KD)
    out = np.empty(B * C * N, dtype=packed.dtype)
    bh, n, d = np.ix_(np.arange(BH), np.arange(N), np.arange(KD))
    b, i = bh // heads, bh % heads
    for j in range(2):
        ch = i * 2 * KD + j * KD + d
        out[_nchw_flat(b, ch, n, C, N)] = packed[2 + j]
    return out.reshape(B, C, H, W)


def merge_attn(o2: np.ndarray, B: int, heads: int, key_dim: int, H: int, W: int) -> np.ndarray:
    """PsaMergeAttn: ``out[b, i*2*KD + j*KD + d, y, x] = o2[j, b*heads+i, n, d]``.

    vision-rs book, "Custom Kernels", "Position-Sensitive Attention (PSA)",
    PsaMergeAttn bullet: the two FA2 outputs (lo, hi) returned to NCHW
    ``[B, c, H, W]`` with c = 2*heads*KEY_DIM.
    """
    KD, N, BH, C = key_dim, H * W, B * heads, 2 * heads * key_dim
    o2 = np.asarray(o2).reshape(2, BH, N, KD)
    out = np.empty(B * C * N, dtype=o2.dtype)
    bh, n, d = np.ix_(np.arange(BH), np.arange(N), np.arange(KD))
    b, i = bh // heads, bh % heads
    for j in range(2):
        ch = i * 2 * KD + j * KD + d
        out[_nchw_flat(b, ch, n, C, N)] = o2[j]
    return out.reshape(B, C, H, W)


def split_attn(out: np.ndarray, B: int, heads: int, key_dim: int, H: int, W: int) -> np.ndarray:
    """Inverse (and adjoint) of :func:`merge_attn`:
    ``o2[j, b*heads+i, n, d] = out[b, i*2*KD + j*KD + d, y, x]``.

    The merge is a permutation, so the gradient reaching its NCHW output goes
    back to the two ``[BH, N, KD]`` halves by the inverse permutation
    (vision-rs book, "Custom Kernels", "Position-Sensitive Attention (PSA)",
    PsaMergeAttn bullet, read backwards).
    """
    KD, N, BH, C = key_dim, H * W, B * heads, 2 * heads * key_dim
    flat = np.asarray(out).reshape(-1)
    assert flat.size == B * C * N, "out has the wrong number of elements"
    bh, n, d = np.ix_(np.arange(BH), np.arange(N), np.arange(KD))
    b, i = bh // heads, bh % heads
    o2 = np.empty((2, BH, N, KD), dtype=flat.dtype)
    for j in range(2):
        o2[j] = flat[_nchw_flat(b, i * 2 * KD + j * KD + d, n, C, N)]
    return o2


def unpack_qkv(packed: np.ndarray, B: int, heads: int, key_dim: int, H: int, W: int) -> np.ndarray:
    """Inverse (and adjoint) of :func:`pack_qkv`:
    ``qkv[b, i*4*KD + s*KD + d, y, x] = packed[s, b*heads+i, n, d]``.

    The pack is a permutation, so gradients with respect to the packed Q, K,
    V_lo, V_hi reach the NCHW QKV tensor by the inverse permutation (vision-rs
    book, "Custom Kernels", "Position-Sensitive Attention (PSA)", PsaPackQkv
    bullet, read backwards).
    """
    KD, N, BH, C = key_dim, H * W, B * heads, 4 * heads * key_dim
    packed = np.asarray(packed).reshape(4, BH, N, KD)
    out = np.empty(B * C * N, dtype=packed.dtype)
    bh, n, d = np.ix_(np.arange(BH), np.arange(N), np.arange(KD))
    b, i = bh // heads, bh % heads
    for s in range(4):
        out[_nchw_flat(b, i * 4 * KD + s * KD + d, n, C, N)] = packed[s]
    return out.reshape(B, C, H, W)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """softmax(scale * Q K^T) V and the row log-sum-exp, per batch-head, in float64.

    vision-rs book, "Custom Kernels", "Flash Attention 2": tensors are
    ``[BATCH*N_HEADS, N_CTX, HEAD_DIM]``; FA2's online softmax computes this
    exactly up to rounding. Returns ``O [BH, n_q, Dv]`` and ``LSE [BH, n_q]``
    with ``LSE = max_m S + ln sum_m exp(S - max)`` (natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    BH, n_q, _ = q.shape
    o = np.empty((BH, n_q, v.shape[2]))
    lse = np.empty((BH, n_q))
    for bh in range(BH):
        s = scale * (q[bh] @ k[bh].T)            # scores [n_q, n_k]
        m = s.max(axis=1, keepdims=True)         # row max
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)         # row sum
        o[bh] = (e / z) @ v[bh]
        lse[bh] = (m + np.log(z))[:, 0]
    return o, lse


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, scale: float):
    """Gradients (dQ, dK, dV) of O = softmax(scale * Q K^T) V, in float64.

    vision-rs book, "Custom Kernels", "Flash Attention 2" names separate dQ and
    dK/dV kernels; the formulas are the standard gradient of the definition in
    :func:`attention`, with P recomputed from the row LSE:
    P = exp(scale*QK^T - LSE), dV = P^T dO, dP = dO V^T,
    Delta = rowsum(dO * O), dS = P * (dP - Delta), dQ = scale*dS K,
    dK = scale*dS^T Q. O and LSE are this oracle's own float64 values.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    o, lse = attention(q, k, v, scale)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for bh in range(q.shape[0]):
        p = np.exp(scale * (q[bh] @ k[bh].T) - lse[bh][:, None])
        dv[bh] = p.T @ dout[bh]
        dp = dout[bh] @ v[bh].T
        delta = (dout[bh] * o[bh]).sum(axis=1)
        ds = p * (dp - delta[:, None])
        dq[bh] = scale * (ds @ k[bh])
        dk[bh] = scale * (ds.T @ q[bh])
    return dq, dk, dv


def psa_forward(qkv: np.ndarray, B: int, heads: int, key_dim: int, H: int, W: int,
                scale: float | None = None):
    """The whole PSA forward: pack, FA2 on (Q, K, V_lo) and (Q, K, V_hi), merge, extract V.

    vision-rs book, "Custom Kernels", "Position-Sensitive Attention (PSA)".
    Returns ``out [B, 2hKD, H, W]``, the V residual ``[B, 2hKD, H, W]`` and
    ``LSE [BH, N]`` (the same for both halves, since they share Q and K).
    """
    if scale is None:
        scale = default_scale(key_dim)
    x = np.asarray(qkv, dtype=np.float64)
    packed = pack_qkv(x, B, heads, key_dim, H, W)
    o_lo, lse = attention(packed[0], packed[1], packed[2], scale)
    o_hi, _ = attention(packed[0], packed[1], packed[3], scale)
    out = merge_attn(np.stack([o_lo, o_hi]), B, heads, key_dim, H, W)
    v_res = extract_v(packed, B, heads, key_dim, H, W)
    return out, v_res, lse


def psa_backward(qkv: np.ndarray, dout: np.ndarray, dv_res, B: int, heads: int, key_dim: int,
                 H: int, W: int, scale: float | None = None) -> np.ndarray:
    """Gradient of the PSA forward with respect to the NCHW QKV tensor, in float64.

    The forward (vision-rs book, "Custom Kernels", "Position-Sensitive
    Attention (PSA)") is pack -> FA2 on (Q, K, V_lo) and on (Q, K, V_hi) ->
    merge, plus extract V for the residual path. Its gradient is the chain
    rule through those steps, taken in reverse:

    * ``dout`` (gradient of ``out``, NCHW ``[B, 2hKD, H, W]``) goes back through
      the merge permutation to the two halves (:func:`split_attn`);
    * each half's FA2 backward (:func:`attention_bwd`, "Flash Attention 2")
      gives dQ_j, dK_j, dV_j; Q and K are shared by both halves, so their
      gradients are the sums dQ_lo + dQ_hi and dK_lo + dK_hi;
    * ``dv_res`` (gradient of the V residual output, NCHW ``[B, 2hKD, H, W]``,
      or None for zero) goes back through the extract permutation and adds to
      dV_lo, dV_hi;
    * the four packed gradients go back through the pack permutation
      (:func:`unpack_qkv`).

    Readings: no gradient flows through the LSE (it is saved state, not an
    output of the block); the scale is KEY_DIM ** -0.5 unless given.
    """
    if scale is None:
        scale = default_scale(key_dim)
    x = np.asarray(qkv, dtype=np.float64)
    packed = pack_qkv(x, B, heads, key_dim, H, W)
    do2 = split_attn(np.asarray(dout, dtype=np.float64), B, heads, key_dim, H, W)
    dq_lo, dk_lo, dv_lo = attention_bwd(packed[0], packed[1], packed[2], do2[0], scale)
    dq_hi, dk_hi, dv_hi = attention_bwd(packed[0], packed[1], packed[3], do2[1], scale)
    dpacked = np.stack([dq_lo + dq_hi, dk_lo + dk_hi, dv_lo, dv_hi])
    if dv_res is not None:
        dpacked[2:] += split_attn(np.asarray(dv_res, dtype=np.float64), B, heads, key_dim, H, W)
    return unpack_qkv(dpacked, B, heads, key_dim, H, W)
