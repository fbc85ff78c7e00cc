"""The PSA backward (psa_attention_bwd: d(qkv) NCHW from dOut and the V-residual gradient)
on the GPU against the float64 oracle."""
import numpy as np
import pytest
import torch

import psa_inputs as I
import vision_transformer_attention_psapackqkv_amd as psa
from oracle import psa_oracle as O
from tests.gpu_helpers import announce, assert_attention_close, device, to_f64

pytestmark = pytest.mark.gpu

# (B, heads, key_dim, H, W): several key and query tiles with ragged tails, every key_dim,
# N a multiple of 8 (tiles staged straight into LDS) and not (staged through registers).
SHAPES = [
    (1, 2, 16, 8, 8),       # N = 64, one tile
    (2, 2, 32, 16, 16),     # N = 256, whole tiles
    (2, 1, 32, 7, 9),       # N = 63
    (1, 2, 64, 10, 13),     # N = 130
    (1, 2, 64, 12, 12),     # N = 144
    (1, 1, 128, 9, 12),     # N = 108
    (1, 1, 16, 1, 1),       # one pixel
    (3, 2, 32, 20, 20),     # N = 400
]


def _id(s):
    return "B{}h{}kd{}_{}x{}".format(*s)


def _inputs(B, h, KD, H, W, seed, with_dv):
    qkv = I.make_qkv(B, h, KD, H, W, seed=seed)
    g = torch.from_numpy(np.random.default_rng(seed + 1).standard_normal((B, 2 * h * KD, H, W)).astype(np.float32))
    dout = g.to(torch.bfloat16)
    dv = None
    if with_dv:
        gv = np.random.default_rng(seed + 2).standard_normal((B, 2 * h * KD, H, W)).astype(np.float32)
        dv = torch.from_numpy(gv).to(torch.bfloat16)
    return qkv, dout, dv


def _run(qkv, dout, dv, h, KD, dev):
    x = qkv.to(dev)
    out, _, lse = psa.psa_attention_fwd(x, h, KD, want_v=False)
    return psa.psa_attention_bwd(x, out, lse, dout.to(dev), h, KD, dv=None if dv is None else dv.to(dev))


@pytest.mark.parametrize("with_dv", [False, True], ids=["no_dv", "dv"])
@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_psa_attention_bwd(shape, with_dv):
    dev = device()
    B, h, KD, H, W = shape
    announce(f"psa_attention_bwd {_id(shape)} dv={with_dv}")
    qkv, dout, dv = _inputs(B, h, KD, H, W, 17 * B + h + KD + H * W, with_dv)
    got = _run(qkv, dout, dv, h, KD, dev)
    want = O.psa_backward(to_f64(qkv), to_f64(dout), None if dv is None else to_f64(dv), B, h, KD, H, W)
    g = to_f64(got).reshape(B, h, 4, KD, H * W)
    wr = want.reshape(B, h, 4, KD, H * W)
    for s, name in enumerate(("dQ", "dK", "dV_lo", "dV_hi")):
        assert_attention_close(g[:, :, s], wr[:, :, s], "bf16", f"psa_attention_bwd {name}")


def test_psa_attention_bwd_40x40():
    """The 40x40 map at full size (B=32, heads=8, key_dim=32: BH=256, N=1600), through the
    launch configuration bench.py times; batch items 0 and 31 (16 heads) against the oracle,
    and on every head the invariant that each K channel's gradient sums to 0 over the map."""
    dev = device()
    B, h, KD, H, W = 32, 8, 32, 40, 40
    announce("psa_attention_bwd 40x40 full size")
    qkv, dout, dv = _inputs(B, h, KD, H, W, 2024, True)
    got = _run(qkv, dout, dv, h, KD, dev)
    g = to_f64(got)
    for b in (0, B - 1):
        want = O.psa_backward(to_f64(qkv[b:b + 1]), to_f64(dout[b:b + 1]), to_f64(dv[b:b + 1]), 1, h, KD, H, W)
        gb = g[b:b + 1].reshape(1, h, 4, KD, H * W)
        wb = want.reshape(1, h, 4, KD, H * W)
        for s, name in enumerate(("dQ", "dK", "dV_lo", "dV_hi")):
            assert_attention_close(gb[:, :, s], wb[:, :, s], "bf16", f"40x40 b={b} {name}")
    ksum = g.reshape(B, h, 4, KD, H * W)[:, :, 1].sum(axis=-1)
    scale = np.abs(g.reshape(B, h, 4, KD, H * W)[:, :, 1]).sum(axis=-1).max()
    assert np.abs(ksum).max() <= 1e-2 * scale, "sum over pixels of dK is not ~0"


def test_psa_attention_bwd_matches_two_fa2_bwd():
    """The fused backward equals the unfused composition built from the library's own calls
    (pack, fa2_bwd per V half, dQ and dK summed) to within bf16 rounding."""
    dev = device()
    B, h, KD, H, W = 2, 2, 32, 12, 12
    announce("psa_attention_bwd vs two fa2_bwd")
    qkv, dout, _ = _inputs(B, h, KD, H, W, 99, False)
    x = qkv.to(dev)
    out, _, lse = psa.psa_attention_fwd(x, h, KD, want_v=False)
    fused = to_f64(psa.psa_attention_bwd(x, out, lse, dout.to(dev), h, KD)).reshape(B, h, 4, KD, H * W)
    N = H * W

    def halves(t):   # NCHW [B, 2hKD, H, W] -> the (lo, hi) halves as contiguous [BH, N, KD]
        r = t.reshape(B, h, 2, KD, N)
        return [r[:, :, j].permute(0, 1, 3, 2).reshape(B * h, N, KD).contiguous() for j in range(2)]

    packed = psa.psa_pack_qkv(x, h, KD)
    o_lo, o_hi = halves(out)
    g_lo, g_hi = halves(dout.to(dev))
    lo = psa.fa2_bwd(packed[0], packed[1], packed[2], o_lo, g_lo, lse)
    hi = psa.fa2_bwd(packed[0], packed[1], packed[3], o_hi, g_hi, lse)

    def nchw(t):   # [BH, N, KD] -> [B, h, KD, N]
        return to_f64(t).reshape(B, h, N, KD).transpose(0, 1, 3, 2)
    ref = [nchw(lo[0]) + nchw(hi[0]), nchw(lo[1]) + nchw(hi[1]), nchw(lo[2]), nchw(hi[2])]
    for s, name in enumerate(("dQ", "dK", "dV_lo", "dV_hi")):
        assert_attention_close(fused[:, :, s], ref[s], "bf16", f"fused vs composed {name}")


def test_psa_attention_bwd_repeatable():
    dev = device()
    B, h, KD, H, W = 1, 2, 64, 16, 16
    announce("psa_attention_bwd repeatable")
    qkv, dout, dv = _inputs(B, h, KD, H, W, 5, True)
    a = _run(qkv, dout, dv, h, KD, dev)
    b = _run(qkv, dout, dv, h, KD, dev)
    assert torch.equal(a, b)


@pytest.mark.parametrize("with_v_grad", [True, False])
def test_autograd_wrapper(with_v_grad):
    """psa_attention (torch autograd over psa_attention_fwd / psa_attention_bwd): its outputs
    equal the forward entry point's bit for bit, qkv.grad equals the backward entry point's
    bit for bit (the V-residual gradient absent when the loss does not use it), and both
    match the oracle."""
    dev = device()
    B, h, KD, H, W = 2, 2, 32, 12, 12
    announce(f"autograd wrapper v_grad={with_v_grad}")
    qkv, dout, dv = _inputs(B, h, KD, H, W, seed=4242, with_dv=with_v_grad)
    x = qkv.to(dev).requires_grad_(True)
    out, v_res = psa.psa_attention(x, h, KD)
    if with_v_grad:
        torch.autograd.backward([out, v_res], [dout.to(dev), dv.to(dev)])
    else:
        out.backward(dout.to(dev))
    out_ref, v_ref, lse = psa.psa_attention_fwd(qkv.to(dev), h, KD)
    dx_ref = psa.psa_attention_bwd(qkv.to(dev), out_ref, lse, dout.to(dev), h, KD,
                                   dv=dv.to(dev) if with_v_grad else None)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), out_ref) and torch.equal(v_res.detach(), v_ref)
    assert torch.equal(x.grad, dx_ref)
    want = O.psa_backward(to_f64(qkv), to_f64(dout), to_f64(dv) if with_v_grad else None, B, h, KD, H, W)
    assert_attention_close(to_f64(x.grad), want, "bf16", "d(qkv) via autograd")


@pytest.mark.parametrize("kd", [16, 32, 64, 128])
def test_psa_attention_bwd_zero_queries(kd):
    """Query channels zero: P is uniform over the N pixels, so the K channels' gradient is
    exactly 0 and each V half's gradient is (1/N) * sum over pixels of that half's dOut, plus
    the V-residual gradient; the Q channels against the oracle."""
    dev = device()
    B, h, H, W = 2, 2, 12, 11
    N = H * W
    announce(f"psa_attention_bwd zero queries kd{kd}")
    qkv, dout, dv = _inputs(B, h, kd, H, W, 80 + kd, True)
    g = qkv.clone().reshape(B, h, 4, kd, N)
    g[:, :, 0] = 0
    qkv = g.reshape(qkv.shape).contiguous()
    got = to_f64(_run(qkv, dout, dv, h, kd, dev)).reshape(B, h, 4, kd, N)
    assert np.abs(got[:, :, 1]).max() == 0.0, "dK is not zero"
    do = to_f64(dout).reshape(B, h, 2, kd, N)
    want_v = np.broadcast_to(do.sum(axis=-1, keepdims=True) / N, do.shape) + to_f64(dv).reshape(B, h, 2, kd, N)
    assert_attention_close(got[:, :, 2:], want_v, "bf16", "dV halves vs (1/N) sum dOut + dV_res")
    want = O.psa_backward(to_f64(qkv), to_f64(dout), to_f64(dv), B, h, kd, H, W).reshape(B, h, 4, kd, N)
    assert_attention_close(got[:, :, 0], want[:, :, 0], "bf16", "dQ vs oracle")


# float32 (PSA_F32): the VALU path, one V half after the other. Every key_dim, N a multiple of
# 8 or not, with and without the V-residual gradient; float32 tolerance against the oracle.
# ... and N = 3 (a pixel's fourth lane sees no query or key) and N = 35 (a second tile of 3)
F32_SHAPES = [(1, 2, 16, 8, 8), (2, 1, 32, 7, 9), (1, 2, 64, 10, 13), (1, 1, 128, 9, 12), (1, 1, 16, 1, 1),
              (2, 1, 32, 1, 3), (1, 2, 64, 5, 7)]


@pytest.mark.parametrize("with_dv", [False, True], ids=["no_dv", "dv"])
@pytest.mark.parametrize("shape", F32_SHAPES, ids=_id)
def test_psa_attention_bwd_f32(shape, with_dv):
    dev = device()
    B, h, KD, H, W = shape
    announce(f"psa_attention_bwd f32 {_id(shape)} dv={with_dv}")
    seed = 23 * B + h + KD + H * W
    qkv = I.make_qkv(B, h, KD, H, W, dtype="f32", dist="uniform", seed=seed)
    rng = np.random.default_rng(seed + 1)
    dout = torch.from_numpy(rng.standard_normal((B, 2 * h * KD, H, W)).astype(np.float32))
    dv = torch.from_numpy(rng.standard_normal((B, 2 * h * KD, H, W)).astype(np.float32)) if with_dv else None
    got = _run(qkv, dout, dv, h, KD, dev)
    assert got.dtype == torch.float32
    want = O.psa_backward(to_f64(qkv), to_f64(dout), None if dv is None else to_f64(dv), B, h, KD, H, W)
    g = to_f64(got).reshape(B, h, 4, KD, H * W)
    wr = want.reshape(B, h, 4, KD, H * W)
    for s, name in enumerate(("dQ", "dK", "dV_lo", "dV_hi")):
        assert_attention_close(g[:, :, s], wr[:, :, s], "f32", f"psa_attention_bwd f32 {name}")


def test_psa_attention_autograd_f32():
    """The autograd op in float32: forward and d(qkv) through the float32 kernels match the
    oracle's forward and backward."""
    dev = device()
    B, h, KD, H, W = 1, 2, 32, 6, 7
    announce("psa_attention autograd f32")
    qkv = I.make_qkv(B, h, KD, H, W, dtype="f32", dist="uniform", seed=123)
    x = qkv.to(dev).requires_grad_()
    out, vres = psa.psa_attention(x, h, KD)
    rng = np.random.default_rng(124)
    g_out = torch.from_numpy(rng.standard_normal(tuple(out.shape)).astype(np.float32)).to(dev)
    g_v = torch.from_numpy(rng.standard_normal(tuple(out.shape)).astype(np.float32)).to(dev)
    torch.autograd.backward([out, vres], [g_out, g_v])
    want_out, _, _ = O.psa_forward(to_f64(qkv), B, h, KD, H, W)
    assert_attention_close(to_f64(out), want_out, "f32", "autograd f32 out")
    want = O.psa_backward(to_f64(qkv), to_f64(g_out), to_f64(g_v), B, h, KD, H, W)
    assert_attention_close(to_f64(x.grad), want, "f32", "autograd f32 d(qkv)")
