"""The seeded input generators: deterministic, right shapes and dtypes (CPU only)."""
import numpy as np
import torch

import psa_inputs as I


def test_workload_shapes():
    w = I.WORKLOADS["psa_fwd_bf16_80x80"]
    assert (w.N, w.BH, w.qkv_channels, w.out_channels) == (6400, 32, 2048, 1024)
    w = I.WORKLOADS["psa_fwd_f32_tiny_8x8"]
    x = I.make_workload_qkv(w)
    assert x.shape == (1, 64, 8, 8) and x.dtype == torch.float32
    assert float(x.abs().max()) <= 1.0


def test_deterministic_and_bf16_rounding():
    a = I.make_qkv(2, 2, 16, 3, 5, dtype="bf16", seed=7)
    b = I.make_qkv(2, 2, 16, 3, 5, dtype="bf16", seed=7)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    f = I.make_qkv(2, 2, 16, 3, 5, dtype="f32", seed=7)
    assert torch.equal(f.to(torch.bfloat16), a)   # bf16 = RNE of the same float32 draw


def test_q_scale_touches_only_query_channels():
    base = I.make_qkv(2, 3, 16, 4, 4, dtype="f32", seed=3)
    peaked = I.make_qkv(2, 3, 16, 4, 4, dtype="f32", seed=3, q_scale=3.0)
    g0 = base.reshape(2, 3, 4, 16, 4, 4)
    g1 = peaked.reshape(2, 3, 4, 16, 4, 4)
    assert torch.equal(g1[:, :, 0], 3.0 * g0[:, :, 0])
    assert torch.equal(g1[:, :, 1:], g0[:, :, 1:])


def test_bwd_inputs_and_views():
    q, k, v, do = I.make_attention_inputs(3, 17, 19, 32, seed=1, with_dout=True)
    assert q.shape == (3, 17, 32) and k.shape == (3, 19, 32) and v.shape == (3, 19, 32) and do.shape == (3, 17, 32)
    bits = I.raw_bits(q)
    assert bits.dtype == np.uint16
    assert np.array_equal(I.as_f64(q), q.to(torch.float64).numpy())


def test_score_ramp_inputs():
    """The ramp generators: deterministic; even queries' dot products climb by score_step per
    key and odd queries' fall, up to the small noise; the NCHW form puts the same kind of rows
    in the query and key channels and leaves V N(0, 1)."""
    step = 0.75
    q, k, v, do = I.make_ramp_attention_inputs(2, 6, 300, 32, score_step=step, seed=9, with_dout=True)
    q2 = I.make_ramp_attention_inputs(2, 6, 300, 32, score_step=step, seed=9)[0]
    assert torch.equal(q, q2) and q.dtype == torch.bfloat16 and do.shape == (2, 6, 32)
    s = torch.einsum("bnd,bmd->bnm", q.double(), k.double())
    m = torch.arange(300, dtype=torch.float64)
    assert (s[:, 0::2] - m * step).abs().max() < 3.0 + 0.02 * 300 * step    # noise plus bf16 rounding
    assert (s[:, 1::2] + m * step).abs().max() < 3.0 + 0.02 * 300 * step
    assert float(do.float().std()) < 0.5                                    # dO ~ N(0, 0.25^2)
    x = I.make_ramp_qkv(1, 2, 16, 5, 6, score_step=step, seed=4)
    g = x.reshape(1, 2, 4, 16, 30).double()
    sc = torch.einsum("bhdn,bhdm->bhnm", g[:, :, 0], g[:, :, 1])           # q_n . k_m per head
    n30 = torch.arange(30, dtype=torch.float64)
    assert (sc[:, :, 0::2] - n30 * step).abs().max() < 3.0
    assert (sc[:, :, 1::2] + n30 * step).abs().max() < 3.0
    assert abs(float(g[:, :, 2:].std()) - 1.0) < 0.2
