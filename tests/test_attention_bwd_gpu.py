"""FA2 backward (Delta, dK/dV, dQ kernels) on the GPU against the float64 oracle."""
import numpy as np
import pytest
import torch

import psa_inputs as I
import vision_transformer_attention_psapackqkv_amd as psa
from oracle import psa_oracle as O
from tests.gpu_helpers import announce, assert_attention_close, device, to_f64

pytestmark = pytest.mark.gpu

# (BH, n_q, n_k, head_dim, dtype): several tiles, ragged tails, every head_dim.
SHAPES = [
    (1, 1, 1, 32, "bf16"),
    (2, 64, 64, 16, "bf16"),
    (3, 100, 77, 32, "bf16"),
    (2, 129, 200, 64, "bf16"),
    (2, 65, 63, 128, "bf16"),
    (4, 300, 260, 32, "bf16"),
    (2, 64, 64, 16, "f32"),
    (3, 100, 77, 32, "f32"),
    (2, 33, 130, 64, "f32"),
    (1, 20, 45, 128, "f32"),
    # float32 with fewer keys or queries than a row's four lanes, and tiles that end after
    # 1..3 of a lane's rows
    (2, 37, 1, 16, "f32"),
    (1, 2, 70, 32, "f32"),
    (2, 3, 5, 64, "f32"),
    (1, 35, 33, 128, "f32"),
]


def _id(s):
    return "BH{}_q{}_k{}_d{}_{}".format(*s)


def _run_bwd(q, k, v, do, dev, o=None, lse=None):
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    if o is None:
        o, lse = psa.fa2_fwd(qd, kd, vd)
    return psa.fa2_bwd(qd, kd, vd, o.to(dev), dod, lse.to(dev))


def _check(grads, q, k, v, do, dt, sel=None):
    qq, kk, vv, gg = (to_f64(t) for t in (q, k, v, do))
    if sel is not None:
        qq, kk, vv, gg = qq[sel], kk[sel], vv[sel], gg[sel]
    want = O.attention_bwd(qq, kk, vv, gg, qq.shape[2] ** -0.5)
    for name, got, w in zip(("dQ", "dK", "dV"), grads, want):
        g = to_f64(got)
        if sel is not None:
            g = g[sel]
        assert_attention_close(g, w, dt, f"fa2_bwd {name}")


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_fa2_bwd(shape):
    dev = device()
    BH, nq, nk, D, dt = shape
    announce(f"fa2_bwd {_id(shape)}")
    q, k, v, do = I.make_attention_inputs(BH, nq, nk, D, dtype=dt, seed=7 * BH + nq + nk + D, with_dout=True)
    grads = _run_bwd(q, k, v, do, dev)
    _check(grads, q, k, v, do, dt)


@pytest.mark.parametrize("shape", SHAPES[:6], ids=_id)
def test_fa2_bwd_from_oracle_forward(shape):
    """O and LSE come from the oracle (O rounded to the storage dtype), isolating the backward."""
    dev = device()
    BH, nq, nk, D, dt = shape
    announce(f"fa2_bwd oracle-fwd {_id(shape)}")
    q, k, v, do = I.make_attention_inputs(BH, nq, nk, D, dtype=dt, seed=3 * BH + nq + nk + D, with_dout=True)
    o64, lse64 = O.attention(to_f64(q), to_f64(k), to_f64(v), D ** -0.5)
    o = torch.from_numpy(o64).to(q.dtype)
    lse = torch.from_numpy(lse64).to(torch.float32)
    grads = _run_bwd(q, k, v, do, dev, o=o, lse=lse)
    _check(grads, q, k, v, do, dt)


def test_fa2_bwd_workload_40x40():
    """The backward workload at full size (BH=256, N=1600, head_dim 32): against the oracle on
    one head of every block of 32 (several per XCD's share of the grid) plus heads 1, 127 and 255,
    and an invariant on every head: sum_m dV[m] = sum_n dO[n]."""
    dev = device()
    w = I.WORKLOADS["fa2_bwd_bf16_40x40"]
    announce("fa2_bwd workload 40x40")
    q, k, v, do = I.make_workload_bwd(w)
    grads = _run_bwd(q, k, v, do, dev)
    sel = np.unique(np.concatenate([np.arange(0, 256, 32), [1, 127, 255]]))
    _check(grads, q, k, v, do, "bf16", sel=sel)
    dv_sum = to_f64(grads[2]).sum(axis=1)
    do_sum = to_f64(do).sum(axis=1)
    # |sum_n dO| is ~40 here; bf16 rounding of P and of each dV element (<= 2^-9 relative)
    # keeps the difference near 1e-2
    assert np.abs(dv_sum - do_sum).max() < 0.1, np.abs(dv_sum - do_sum).max()


@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_fa2_bwd_zero_queries(D):
    """Q = 0: every P row is uniform (1/n_k), so dV[m] = (1/n_k) * sum_n dO[n] for every key m
    and dK = scale * dS^T Q = 0 exactly; dQ against the oracle."""
    dev = device()
    BH, nq, nk = 3, 150, 200
    announce(f"fa2_bwd zero queries d{D}")
    q, k, v, do = I.make_attention_inputs(BH, nq, nk, D, seed=70 + D, with_dout=True)
    q = torch.zeros_like(q)
    dq, dk, dv = _run_bwd(q, k, v, do, dev)
    want_dv = np.broadcast_to(to_f64(do).sum(axis=1, keepdims=True) / nk, (BH, nk, D))
    assert_attention_close(to_f64(dv), want_dv, "bf16", "dV vs (1/n_k) sum dO")
    assert float(dk.float().abs().max()) == 0.0, "dK is not zero"
    _check((dq, dk, dv), q, k, v, do, "bf16")


def test_fa2_f32_more_batch_heads_than_one_launch():
    """float32 fa2_fwd and fa2_bwd with 2^22 + 3 batch-heads of 128 queries: four lanes per
    query make 2^31 + 1,536 work-items in the forward and dQ kernels, so each is split into two
    launches by batch-head (the second covers the last three). Inputs are drawn on the GPU (~150 GB
    in all); the first, a middle and the last three batch-heads are checked against the oracle."""
    dev = device()
    BH, nq, nk, D = (1 << 22) + 3, 128, 5, 16
    announce(f"fa2 f32 BH={BH} q{nq} k{nk} d{D}: two launches per kernel")
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    q, k, v, do = (torch.rand(shape, generator=g, device=dev).mul_(2).sub_(1)
                   for shape in ((BH, nq, D), (BH, nk, D), (BH, nk, D), (BH, nq, D)))
    s = D ** -0.5
    o, lse = psa.fa2_fwd(q, k, v, scale=s)
    dq, dk, dv = psa.fa2_bwd(q, k, v, o, do, lse, scale=s)
    torch.cuda.synchronize()
    sel = torch.tensor([0, BH // 2, BH - 3, BH - 2, BH - 1], device=dev)
    pick = lambda t: to_f64(t.index_select(0, sel))
    want_o, want_lse = O.attention(pick(q), pick(k), pick(v), s)
    assert_attention_close(pick(o), want_o, "f32", "fa2_fwd O, sampled batch-heads")
    assert np.abs(pick(lse) - want_lse).max() < 1e-4
    want = O.attention_bwd(pick(q), pick(k), pick(v), pick(do), s)
    for name, got, w in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        assert_attention_close(pick(got), w, "f32", f"fa2_bwd {name}, sampled batch-heads")
