"""Checks that pin the CPU oracle to facts other than itself.

Each ``check_*`` takes the oracle function(s) as arguments and raises
AssertionError when a fact fails, so the same checks can be run on the real
oracle (must pass) and on copies with a planted mistake (must fail). The facts
are closed forms of softmax attention, invariants, a hand-worked example and
routes through library routines (numpy reshape/transpose, torch SDPA/autograd)
that share no code with the oracle.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- layout

def check_pack(pack_qkv):
    # 1) a library route: the channel axis splits as (head, slot, d), the map flattens
    #    row-major, then axes are permuted to (slot, batch*head, n, d).
    for (B, h, KD, H, W) in [(2, 3, 4, 2, 5), (1, 1, 16, 8, 8), (3, 2, 2, 1, 1)]:
        qkv = _rng(B * 100 + h).integers(0, 2**31, size=(B, 4 * h * KD, H, W), dtype=np.int64)
        want = qkv.reshape(B, h, 4, KD, H * W).transpose(2, 0, 1, 4, 3).reshape(4, B * h, H * W, KD)
        got = pack_qkv(qkv, B, h, KD, H, W)
        assert got.shape == (4, B * h, H * W, KD), "pack: wrong output shape"
        assert np.array_equal(got, want), "pack: disagrees with the reshape/transpose route"
    # 2) brute force on unique ids: decode every packed element back to (b, ch, y, x).
    B, h, KD, H, W = 2, 2, 3, 2, 3
    C, N = 4 * h * KD, H * W
    ids = np.arange(B * C * N, dtype=np.int64).reshape(B, C, H, W)
    got = pack_qkv(ids, B, h, KD, H, W)
    seen = set()
    for s in range(4):
        for bh in range(B * h):
            for n in range(N):
                for d in range(KD):
                    v = int(got[s, bh, n, d])
                    seen.add(v)
                    b, rem = divmod(v, C * N)
                    ch, pos = divmod(rem, N)
                    y, x = divmod(pos, W)
                    assert b == bh // h and y * W + x == n, "pack: wrong batch or position"
                    assert ch == (bh % h) * 4 * KD + s * KD + d, "pack: wrong channel"
    assert len(seen) == B * C * N, "pack: not a permutation"


def check_extract(pack_qkv, extract_v):
    for (B, h, KD, H, W) in [(2, 3, 4, 2, 5), (1, 2, 8, 3, 1)]:
        qkv = _rng(7 + B).integers(0, 2**31, size=(B, 4 * h * KD, H, W), dtype=np.int64)
        # the V section of each head group, picked by a channel slice of the input
        want = qkv.reshape(B, h, 4, KD, H, W)[:, :, 2:4].reshape(B, 2 * h * KD, H, W)
        got = extract_v(pack_qkv(qkv, B, h, KD, H, W), B, h, KD, H, W)
        assert got.shape == want.shape and np.array_equal(got, want), \
            "extract: pack then extract does not return the V channels"


def check_merge(merge_attn):
    for (B, h, KD, H, W) in [(2, 3, 4, 2, 5), (1, 1, 16, 8, 8)]:
        o2 = _rng(11 + h).integers(0, 2**31, size=(2, B * h, H * W, KD), dtype=np.int64)
        want = o2.reshape(2, B, h, H * W, KD).transpose(1, 2, 0, 4, 3).reshape(B, 2 * h * KD, H, W)
        got = merge_attn(o2, B, h, KD, H, W)
        assert got.shape == want.shape and np.array_equal(got, want), \
            "merge: disagrees with the reshape/transpose route"
        # inverse: split channels as (head, half, d) and flatten the map back
        back = got.reshape(B, h, 2, KD, H * W).transpose(2, 0, 1, 4, 3).reshape(2, B * h, H * W, KD)
        assert np.array_equal(back, o2), "merge: not invertible by the channel split"


# ------------------------------------------------------------------------ attention

def _sdpa_torch(q, k, v, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    lse = torch.logsumexp(scale * (qt @ kt.transpose(-1, -2)), dim=-1)
    return o.numpy(), lse.numpy()


def check_attention(attention):
    rng = _rng(3)
    # closed form: Q = 0 gives uniform rows, O = mean(V), LSE = ln N
    q = np.zeros((2, 5, 4)); k = rng.normal(size=(2, 7, 4)); v = rng.normal(size=(2, 7, 3))
    o, lse = attention(q, k, v, 0.5)
    assert np.allclose(o, v.mean(axis=1, keepdims=True).repeat(5, axis=1), atol=1e-12), "Q=0: O != mean(V)"
    assert np.allclose(lse, math.log(7), atol=1e-12), "Q=0: LSE != ln N"
    # closed form: one key gives O = V, LSE = s q.k
    q = rng.normal(size=(3, 4, 6)); k = rng.normal(size=(3, 1, 6)); v = rng.normal(size=(3, 1, 5))
    o, lse = attention(q, k, v, 0.3)
    assert np.allclose(o, np.repeat(v, 4, axis=1), atol=1e-12), "N=1: O != V"
    assert np.allclose(lse, 0.3 * np.einsum("bnd,bd->bn", q, k[:, 0]), atol=1e-12), "N=1: LSE != s q.k"
    # closed form: two keys give a logistic mix, LSE = s q.k1 + ln(1 + e^(s q.(k0-k1)))
    q = rng.normal(size=(2, 6, 3)); k = rng.normal(size=(2, 2, 3)); v = rng.normal(size=(2, 2, 4))
    s = 0.7
    o, lse = attention(q, k, v, s)
    t = s * np.einsum("bnd,bd->bn", q, k[:, 0] - k[:, 1])
    w0 = 1.0 / (1.0 + np.exp(-t))
    want = w0[..., None] * v[:, None, 0] + (1.0 - w0)[..., None] * v[:, None, 1]
    assert np.allclose(o, want, atol=1e-12), "N=2: not the logistic mix"
    want_lse = s * np.einsum("bnd,bd->bn", q, k[:, 1]) + np.log1p(np.exp(t))
    assert np.allclose(lse, want_lse, atol=1e-12), "N=2: wrong LSE"
    # rows of the attention matrix are a probability distribution (V = identity)
    q = rng.normal(size=(2, 9, 4)); k = rng.normal(size=(2, 11, 4))
    p, _ = attention(q, k, np.broadcast_to(np.eye(11), (2, 11, 11)).copy(), 0.9)
    assert np.all(p >= 0) and np.allclose(p.sum(axis=2), 1.0, atol=1e-12), "rows do not sum to 1"
    # a query that matches one key much better puts its weight there
    assert np.allclose(p.argmax(axis=2), np.argmax(np.einsum("bnd,bmd->bnm", q, k), axis=2)), "argmax moved"
    # joint permutation of keys and values changes nothing
    v = rng.normal(size=(2, 11, 5))
    perm = rng.permutation(11)
    o1, l1 = attention(q, k, v, 0.9)
    o2, l2 = attention(q, k[:, perm], v[:, perm], 0.9)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12), "not permutation invariant"
    # a key offset u adds s q.u to every score of a row: O unchanged, LSE shifted
    u = rng.normal(size=4)
    o3, l3 = attention(q, k + u, v, 0.9)
    assert np.allclose(o1, o3, atol=1e-11), "K + u changed O"
    assert np.allclose(l3, l1 + 0.9 * np.einsum("bnd,d->bn", q, u), atol=1e-11), "K + u: wrong LSE shift"
    # linear in V
    v2 = rng.normal(size=(2, 11, 5))
    oa, _ = attention(q, k, 2.0 * v - 3.0 * v2, 0.9)
    ob, _ = attention(q, k, v2, 0.9)
    assert np.allclose(oa, 2.0 * o1 - 3.0 * ob, atol=1e-11), "not linear in V"
    # two halves of V give the halves of one attention over [V_lo | V_hi]
    vl, vh = rng.normal(size=(2, 11, 4)), rng.normal(size=(2, 11, 4))
    olo, llo = attention(q, k, vl, 0.5)
    ohi, lhi = attention(q, k, vh, 0.5)
    ocat, lcat = attention(q, k, np.concatenate([vl, vh], axis=2), 0.5)
    assert np.allclose(np.concatenate([olo, ohi], axis=2), ocat, atol=1e-12), "halves != head_dim 2KD"
    assert np.allclose(llo, lcat) and np.allclose(lhi, lcat), "halves: LSE differs"
    # large scores (one near 900, past exp's float64 range): finite and equal to torch's result
    kk = rng.normal(size=(1, 8, 4)); vv = rng.normal(size=(1, 8, 3))
    big_q = 5.0 * rng.normal(size=(1, 8, 4))
    big_q[0, 0] = 900.0 * kk[0, 0] / (kk[0, 0] @ kk[0, 0])
    ob1, lb1 = attention(big_q, kk, vv, 1.0)
    assert np.all(np.isfinite(ob1)) and np.all(np.isfinite(lb1)), "overflow at large scores"
    to1, tl1 = _sdpa_torch(big_q, kk, vv, 1.0)
    assert np.allclose(ob1, to1, atol=1e-9) and np.allclose(lb1, tl1, atol=1e-9), "large scores: wrong result"
    # library routine: torch CPU float64 scaled_dot_product_attention
    for (BH, nq, nk, D, Dv, s) in [(3, 17, 13, 8, 8, 8 ** -0.5), (2, 40, 64, 16, 32, 0.25)]:
        q = rng.normal(size=(BH, nq, D)); k = rng.normal(size=(BH, nk, D)); v = rng.normal(size=(BH, nk, Dv))
        o, lse = attention(q, k, v, s)
        to, tl = _sdpa_torch(q, k, v, s)
        assert np.allclose(o, to, atol=1e-12, rtol=0), "disagrees with torch SDPA"
        assert np.allclose(lse, tl, atol=1e-12, rtol=0), "LSE disagrees with torch logsumexp"


def check_psa_golden(psa_forward, pack_qkv):
    with open(os.path.join(GOLDEN, "psa_two_head_worked.json")) as f:
        g = json.load(f)
    qkv = np.array(g["qkv"], dtype=np.float64)
    dims = (g["B"], g["heads"], g["key_dim"], g["H"], g["W"])
    assert np.array_equal(pack_qkv(qkv, *dims), np.array(g["packed"])), "golden: packed layout"
    out, v, lse = psa_forward(qkv, *dims)
    assert np.allclose(out, np.array(g["out"]), atol=1e-12, rtol=0), "golden: out"
    assert np.array_equal(v, np.array(g["v"])), "golden: V residual"
    assert np.allclose(lse, np.array(g["lse"]), atol=1e-12, rtol=0), "golden: LSE"
    # the default scale is KEY_DIM ** -0.5: an explicit 0.5 gives the same result
    out2, _, _ = psa_forward(qkv, *dims, scale=g["scale"])
    assert np.allclose(out, out2, atol=0, rtol=0), "golden: default scale is not KEY_DIM**-0.5"


# ------------------------------------------------------------------------- backward

def _loss(attention, q, k, v, g, s):
    o, _ = attention(q, k, v, s)
    return float((o * g).sum())


def check_attention_bwd(attention_bwd, attention):
    rng = _rng(5)
    s = 0.6
    q = rng.normal(size=(2, 4, 3)); k = rng.normal(size=(2, 5, 3)); v = rng.normal(size=(2, 5, 2))
    g = rng.normal(size=(2, 4, 2))
    dq, dk, dv = attention_bwd(q, k, v, g, s)
    # central finite differences of L = sum(O * dO)
    eps = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps; lp = _loss(attention, q, k, v, g, s)
            x[idx] = old - eps; lm = _loss(attention, q, k, v, g, s)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        assert np.allclose(dx, num, atol=1e-8, rtol=1e-6), "backward disagrees with finite differences"
    # torch float64 autograd through an explicit softmax
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    p = torch.softmax(s * tq @ tk.transpose(-1, -2), dim=-1)
    (p @ tv).backward(torch.tensor(g))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(mine, ref.numpy(), atol=1e-12, rtol=0), "backward disagrees with torch autograd"
    # invariants: sum over keys of dK is 0 (K -> K + u leaves O unchanged);
    # sum over keys of dV equals sum over queries of dO (rows of P sum to 1)
    q = rng.normal(size=(3, 7, 4)); k = rng.normal(size=(3, 9, 4)); v = rng.normal(size=(3, 9, 5))
    g = rng.normal(size=(3, 7, 5))
    _, dk, dv = attention_bwd(q, k, v, g, 0.5)
    assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-12), "sum_m dK != 0"
    assert np.allclose(dv.sum(axis=1), g.sum(axis=1), atol=1e-12), "sum_m dV != sum_n dO"
    # Q = 0: every P entry is 1/N_k, so dV[m] = (1/N_k) sum_n dO[n] for every key m
    _, _, dv0 = attention_bwd(np.zeros_like(q), k, v, g, 0.5)
    assert np.allclose(dv0, np.repeat(g.sum(axis=1, keepdims=True) / 9.0, 9, axis=1), atol=1e-12), "Q=0: dV"


# --------------------------------------------------------------------- PSA backward

def _psa_torch(x, B, h, KD, H, W, s):
    """The PSA forward written with torch reshapes (a route independent of the oracle):
    channels split as (head, slot, d), the map flattened row-major."""
    t = x.reshape(B, h, 4, KD, H * W)
    q = t[:, :, 0].transpose(-1, -2)
    k = t[:, :, 1].transpose(-1, -2)
    v = torch.cat([t[:, :, 2], t[:, :, 3]], dim=2).transpose(-1, -2)      # [B, h, N, 2KD]
    p = torch.softmax(s * q @ k.transpose(-1, -2), dim=-1)
    out = (p @ v).transpose(-1, -2).reshape(B, 2 * h * KD, H, W)
    vres = t[:, :, 2:4].reshape(B, 2 * h * KD, H, W)
    return out, vres


def check_psa_backward(psa_backward, psa_forward):
    rng = _rng(11)
    # 1) central finite differences of L = <dout, out> + <dvres, v_res> through the forward
    B, h, KD, H, W = 1, 2, 2, 2, 2
    s = 0.7
    x = rng.normal(size=(B, 4 * h * KD, H, W))
    g = rng.normal(size=(B, 2 * h * KD, H, W))
    gv = rng.normal(size=(B, 2 * h * KD, H, W))

    def loss(xx):
        out, vres, _ = psa_forward(xx, B, h, KD, H, W, s)
        return float((out * g).sum() + (vres * gv).sum())

    dx = psa_backward(x, g, gv, B, h, KD, H, W, s)
    assert dx.shape == x.shape, "d(qkv) has the wrong shape"
    eps = 1e-6
    num = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        old = x[idx]
        x[idx] = old + eps; lp = loss(x)
        x[idx] = old - eps; lm = loss(x)
        x[idx] = old
        num[idx] = (lp - lm) / (2 * eps)
    assert np.allclose(dx, num, atol=1e-8, rtol=1e-6), "PSA backward disagrees with finite differences"
    # 2) torch float64 autograd through the torch-written forward, larger shapes
    B, h, KD, H, W = 2, 3, 4, 3, 5
    s = KD ** -0.5
    x = rng.normal(size=(B, 4 * h * KD, H, W))
    g = rng.normal(size=(B, 2 * h * KD, H, W))
    gv = rng.normal(size=(B, 2 * h * KD, H, W))
    tx = torch.tensor(x, requires_grad=True)
    out, vres = _psa_torch(tx, B, h, KD, H, W, s)
    ((out * torch.tensor(g)).sum() + (vres * torch.tensor(gv)).sum()).backward()
    dx = psa_backward(x, g, gv, B, h, KD, H, W, s)
    assert np.allclose(dx, tx.grad.numpy(), atol=1e-11, rtol=0), "PSA backward disagrees with torch autograd"
    # without the residual gradient (None) it equals the gradient of <dout, out> alone
    tx.grad = None
    out, _ = _psa_torch(tx, B, h, KD, H, W, s)
    (out * torch.tensor(g)).sum().backward()
    dx0 = psa_backward(x, g, None, B, h, KD, H, W, None)
    assert np.allclose(dx0, tx.grad.numpy(), atol=1e-11, rtol=0), "PSA backward without dv_res"
    # 3) invariants per head: K channels' gradient sums to 0 over the map (K -> K + u leaves
    #    the output unchanged); V channels' gradient sums to the map-sum of dout (+ dv_res),
    #    since the rows of P sum to 1
    dxr = dx.reshape(B, h, 4, KD, H * W)
    assert np.allclose(dxr[:, :, 1].sum(axis=-1), 0.0, atol=1e-11), "sum over pixels of dK != 0"
    gr = (g + gv).reshape(B, h, 2, KD, H * W).sum(axis=-1)
    assert np.allclose(dxr[:, :, 2:4].sum(axis=-1), gr, atol=1e-11), "sum over pixels of dV"
