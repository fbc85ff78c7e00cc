"""Seeded random shapes through the fused PSA forward and backward and through FA2 forward
and backward, each against the float64 oracle.

The shapes are drawn once from a fixed seed (so the list is the same on every run), over
every key/head dim, maps and sequence lengths that are and are not multiples of the tile
sizes and of 8 (the directly staged and the register-staged kernels), and n_q != n_k; the PSA
maps in bf16 and, from a second draw, in float32.
"""
import numpy as np
import pytest
import torch

import psa_inputs as I
import vision_transformer_attention_psapackqkv_amd as psa
from oracle import psa_oracle as O
from tests.gpu_helpers import announce, assert_attention_close, assert_lse_close, bits, device, to_f64

pytestmark = pytest.mark.gpu


def _psa_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        KD = int(rng.choice([16, 32, 64, 128]))
        B, h = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        H, W = int(rng.integers(1, 31)), int(rng.integers(1, 31))
        out.append((B, h, KD, H, W))
    return out


def _fa2_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        D = int(rng.choice([16, 32, 64, 128]))
        BH = int(rng.integers(1, 7))
        nq, nk = int(rng.integers(1, 700)), int(rng.integers(1, 700))
        dt = "f32" if rng.random() < 0.25 else "bf16"
        out.append((BH, nq, nk, D, dt))
    return out


PSA_RANDOM = _psa_shapes(12, 2026)
FA2_RANDOM = _fa2_shapes(12, 2027)


def _psa_id(s):
    return "B{}h{}kd{}_{}x{}".format(*s)


# float32 maps (the VALU kernels, four lanes per row) drawn the same way from another seed
PSA_RANDOM_F32 = _psa_shapes(6, 2028)
PSA_CASES = [(s, "bf16") for s in PSA_RANDOM] + [(s, "f32") for s in PSA_RANDOM_F32]


@pytest.mark.parametrize("case", PSA_CASES, ids=lambda c: _psa_id(c[0]) + "_" + c[1])
def test_random_psa_fwd_bwd(case):
    dev = device()
    shape, dt = case
    B, h, KD, H, W = shape
    announce(f"random psa fwd/bwd {_psa_id(shape)} {dt}")
    seed = 7000 + B * 1000 + h * 100 + KD + H * W
    qkv = I.make_qkv(B, h, KD, H, W, dtype=dt, seed=seed)
    x = qkv.to(dev)
    out, vres, lse = psa.psa_attention_fwd(x, h, KD)
    want_out, _, want_lse = O.psa_forward(to_f64(qkv), B, h, KD, H, W)
    assert_attention_close(to_f64(out), want_out, dt, "random psa_attention_fwd out")
    assert_lse_close(to_f64(lse), want_lse, dt, "random psa_attention_fwd")
    want_v = O.extract_v(O.pack_qkv(bits(qkv), B, h, KD, H, W), B, h, KD, H, W)
    assert np.array_equal(bits(vres), want_v), "V residual differs"

    rng = np.random.default_rng(seed + 1)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dout = torch.from_numpy(rng.standard_normal(tuple(out.shape)).astype(np.float32)).to(tdt)
    dv = torch.from_numpy(rng.standard_normal(tuple(out.shape)).astype(np.float32)).to(tdt)
    got = to_f64(psa.psa_attention_bwd(x, out, lse, dout.to(dev), h, KD, dv=dv.to(dev)))
    want = O.psa_backward(to_f64(qkv), to_f64(dout), to_f64(dv), B, h, KD, H, W)
    g = got.reshape(B, h, 4, KD, H * W)
    wr = want.reshape(B, h, 4, KD, H * W)
    for s, name in enumerate(("dQ", "dK", "dV_lo", "dV_hi")):
        assert_attention_close(g[:, :, s], wr[:, :, s], dt, f"random psa_attention_bwd {name}")


@pytest.mark.parametrize("shape", FA2_RANDOM, ids=lambda s: "BH{}_q{}_k{}_d{}_{}".format(*s))
def test_random_fa2_fwd_bwd(shape):
    dev = device()
    BH, nq, nk, D, dt = shape
    announce(f"random fa2 fwd/bwd BH{BH} q{nq} k{nk} d{D} {dt}")
    q, k, v, do = I.make_attention_inputs(BH, nq, nk, D, dtype=dt, seed=8000 + BH + nq + nk + D,
                                          with_dout=True)
    # dK and dV sum over the queries: with n_q >> n_k they grow like sqrt(n_q / n_k), and a
    # bf16 value above ~5 rounds by more than the absolute tolerance on storage alone; dO is
    # scaled so that the gradients stay O(1), which is what the tolerance presumes.
    f = min(1.0, (nk / nq) ** 0.5)
    if f < 1.0:
        do = (do.float() * f).to(do.dtype)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    s = D ** -0.5
    o, lse = psa.fa2_fwd(qd, kd, vd)
    want_o, want_lse = O.attention(to_f64(q), to_f64(k), to_f64(v), s)
    assert_attention_close(to_f64(o), want_o, dt, "random fa2_fwd O")
    assert_lse_close(to_f64(lse), want_lse, dt, "random fa2_fwd")
    grads = psa.fa2_bwd(qd, kd, vd, o, dod, lse)
    want = O.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), s)
    for name, got, w in zip(("dQ", "dK", "dV"), grads, want):
        assert_attention_close(to_f64(got), w, dt, f"random fa2_bwd {name}")
