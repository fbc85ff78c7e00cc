"""The binding rejects mis-sized, mis-typed and misplaced tensors before anything is allocated
or launched (ValueError), for every tensor each entry point hands to the C ABI.

Host logic only: the check that a tensor lives on the GPU is replaced by one that accepts CPU
tensors, so each call below reaches exactly the one check it is meant to fail; none of them can
get as far as a launch (the next step would need a GPU stream and raise something else)."""
import pytest
import torch

import vision_transformer_attention_psapackqkv_amd as psa
from vision_transformer_attention_psapackqkv_amd import _binding as b

BF = torch.bfloat16
F32 = torch.float32


@pytest.fixture(autouse=True)
def cpu_ok(monkeypatch):
    def dev(t, name):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t
    monkeypatch.setattr(b, "_dev", dev)

    def no_stream(_t):
        raise AssertionError("a call with a bad argument reached the launch")
    monkeypatch.setattr(b, "_stream", no_stream)


def e(*shape, dtype=BF):
    return torch.empty(shape, dtype=dtype)


def expect(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


B, h, KD, H, W = 2, 2, 16, 4, 6
N, BH = H * W, B * h


def test_pack_checks():
    expect("channels", psa.psa_pack_qkv, e(B, 4 * h * KD + 1, H, W), h, KD)
    expect("4-D", psa.psa_pack_qkv, e(B, 4 * h * KD, N), h, KD)
    expect("dtype", psa.psa_pack_qkv, e(B, 4 * h * KD, H, W, dtype=torch.float16), h, KD)
    expect("out has shape", psa.psa_pack_qkv, e(B, 4 * h * KD, H, W), h, KD, out=e(4, BH, N, KD - 1))
    expect("out has dtype", psa.psa_pack_qkv, e(B, 4 * h * KD, H, W), h, KD, out=e(4, BH, N, KD, dtype=F32))
    expect("contiguous", psa.psa_pack_qkv, e(B, 4 * h * KD, H, W), h, KD,
           out=e(4, BH, KD, N).transpose(2, 3))


@pytest.mark.parametrize("fn,slots", [(psa.psa_merge_attn, 2), (psa.psa_extract_v, 4)])
def test_merge_extract_checks(fn, slots):
    expect("input has shape", fn, e(slots + 1, BH, N, KD), B, h, KD, H, W)
    expect("input has dtype", fn, e(slots, BH, N, KD, dtype=torch.int16), B, h, KD, H, W)
    expect("out has shape", fn, e(slots, BH, N, KD), B, h, KD, H, W, out=e(B, 2 * h * KD, H, W + 1))
    expect("out has dtype", fn, e(slots, BH, N, KD), B, h, KD, H, W, out=e(B, 2 * h * KD, H, W, dtype=F32))


def test_fa2_fwd_checks():
    q, k = e(BH, 40, 32), e(BH, 24, 32)
    expect("q must be a 3-D", psa.fa2_fwd, e(BH, 40), k, k)
    expect("k has shape", psa.fa2_fwd, q, e(BH + 1, 24, 32), k)
    expect("v has shape", psa.fa2_fwd, q, k, e(BH, 23, 32))
    expect("k has dtype", psa.fa2_fwd, q, e(BH, 24, 32, dtype=F32), k)
    expect("out has shape", psa.fa2_fwd, q, k, k, out=e(BH, 24, 32))
    expect("out has dtype", psa.fa2_fwd, q, k, k, out=e(BH, 40, 32, dtype=F32))
    expect("lse has shape", psa.fa2_fwd, q, k, k, lse=e(BH, 24, dtype=F32))
    expect("lse has dtype", psa.fa2_fwd, q, k, k, lse=e(BH, 40))


def test_fa2_bwd_checks():
    q, k = e(BH, 40, 32), e(BH, 24, 32)
    lse = e(BH, 40, dtype=F32)
    expect("o has shape", psa.fa2_bwd, q, k, k, e(BH, 24, 32), q, lse)
    expect("o has dtype", psa.fa2_bwd, q, k, k, e(BH, 40, 32, dtype=F32), q, lse)
    expect("dout has shape", psa.fa2_bwd, q, k, k, q, e(BH, 40, 16), lse)
    expect("dout has dtype", psa.fa2_bwd, q, k, k, q, e(BH, 40, 32, dtype=F32), lse)
    expect("lse has shape", psa.fa2_bwd, q, k, k, q, q, e(BH, 24, dtype=F32))
    expect("lse has dtype", psa.fa2_bwd, q, k, k, q, q, e(BH, 40))
    expect("workspace holds", psa.fa2_bwd, q, k, k, q, q, lse, workspace=e(BH * 40 - 1, dtype=F32))


def test_psa_fwd_checks():
    x = e(B, 4 * h * KD, H, W)
    shape = (B, 2 * h * KD, H, W)
    expect("channels", psa.psa_attention_fwd, e(B, 4 * h * KD - 8, H, W), h, KD)
    expect("out has shape", psa.psa_attention_fwd, x, h, KD, out=e(B, 2 * h * KD, H, W - 1))
    expect("out has dtype", psa.psa_attention_fwd, x, h, KD, out=e(*shape, dtype=F32))
    expect("v_out has shape", psa.psa_attention_fwd, x, h, KD, out=e(*shape), v_out=e(B, h * KD, H, W))
    expect("v_out has dtype", psa.psa_attention_fwd, x, h, KD, out=e(*shape), v_out=e(*shape, dtype=F32))
    expect("lse has shape", psa.psa_attention_fwd, x, h, KD, out=e(*shape), v_out=e(*shape),
           lse=e(BH, N + 1, dtype=F32))
    expect("lse has dtype", psa.psa_attention_fwd, x, h, KD, out=e(*shape), v_out=e(*shape), lse=e(BH, N))


def test_psa_bwd_checks():
    x = e(B, 4 * h * KD, H, W)
    shape = (B, 2 * h * KD, H, W)
    o, lse = e(*shape), e(BH, N, dtype=F32)
    expect("out has shape", psa.psa_attention_bwd, x, e(B, h * KD, H, W), lse, o, h, KD)
    expect("lse has shape", psa.psa_attention_bwd, x, o, e(BH, N - 1, dtype=F32), o, h, KD)
    expect("lse has dtype", psa.psa_attention_bwd, x, o, e(BH, N), o, h, KD)
    expect("dout has shape", psa.psa_attention_bwd, x, o, lse, e(B, 2 * h * KD, H + 1, W), h, KD)
    expect("dout has dtype", psa.psa_attention_bwd, x, o, lse, e(*shape, dtype=F32), h, KD)
    expect("dv has shape", psa.psa_attention_bwd, x, o, lse, o, h, KD, dv=e(B, 2 * h * KD, H, W + 1))
    expect("dqkv has shape", psa.psa_attention_bwd, x, o, lse, o, h, KD, dqkv=e(*shape))
    expect("dqkv has dtype", psa.psa_attention_bwd, x, o, lse, o, h, KD, dqkv=e(*x.shape, dtype=F32))
    need = b.load_library().psa_attention_bwd_workspace_bytes(B, h, H, W)
    expect("workspace holds", psa.psa_attention_bwd, x, o, lse, o, h, KD,
           workspace=e(need - 1, dtype=torch.uint8))
