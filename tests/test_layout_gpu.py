"""PsaPackQkv, PsaExtractV and PsaMergeAttn on the GPU: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import psa_inputs as I
import vision_transformer_attention_psapackqkv_amd as psa
from oracle import psa_oracle as O
from tests.gpu_helpers import announce, bits, device

pytestmark = pytest.mark.gpu

# (B, heads, key_dim, H, W, dtype): the workload maps, then ragged pixel counts
# (N = 1, 7, 63, 65, 400 and N not a multiple of 8 or 4) at every key_dim, then
# ragged staged tiles.
SHAPES = [
    (1, 1, 16, 8, 8, "f32"),
    (8, 4, 32, 20, 20, "bf16"),
    (2, 3, 16, 1, 1, "bf16"),
    (2, 2, 32, 1, 7, "bf16"),
    (1, 2, 64, 7, 9, "bf16"),
    (3, 1, 128, 5, 13, "bf16"),
    (2, 2, 16, 20, 20, "f32"),
    (1, 3, 32, 3, 5, "f32"),
    (2, 1, 64, 2, 2, "f32"),
    (1, 1, 128, 9, 7, "f32"),
    (2, 2, 64, 16, 16, "bf16"),
    # N a multiple of 8 (4 for f32) but not of the staged tile's pixel count
    # (tile bytes / (key_dim * element size); 16 KB tiles for pack, 8 KB for
    # merge and extract below key_dim 128): several tiles and a short last one.
    (2, 1, 128, 8, 10, "bf16"),
    (1, 2, 128, 12, 12, "f32"),
    (2, 2, 16, 24, 24, "bf16"),
    (1, 1, 32, 12, 12, "f32"),
    (1, 2, 64, 9, 24, "bf16"),
]


def _ids(shape):
    return "B{}h{}kd{}_{}x{}_{}".format(*shape)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_pack_extract_merge_bit_exact(shape):
    dev = device()
    B, h, KD, H, W, dt = shape
    announce(f"layout {_ids(shape)}")
    qkv = I.make_qkv(B, h, KD, H, W, dtype=dt, seed=B * 1000 + h * 100 + KD + H * W)
    packed = psa.psa_pack_qkv(qkv.to(dev), h, KD)
    want_packed = O.pack_qkv(bits(qkv), B, h, KD, H, W)
    assert np.array_equal(bits(packed), want_packed), "pack differs"
    v = psa.psa_extract_v(packed, B, h, KD, H, W)
    assert np.array_equal(bits(v), O.extract_v(want_packed, B, h, KD, H, W)), "extract differs"
    o2 = I.make_attention_inputs(2, B * h * H * W, 1, KD, dtype=dt, seed=5)[0].reshape(2, B * h, H * W, KD)
    merged = psa.psa_merge_attn(o2.to(dev), B, h, KD, H, W)
    assert np.array_equal(bits(merged), O.merge_attn(bits(o2), B, h, KD, H, W)), "merge differs"
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_iota_patterns(dt):
    """Every element carries its own index (16-bit: two passes, low and high half)."""
    dev = device()
    B, h, KD, H, W = 2, 3, 32, 9, 8
    n = B * 4 * h * KD * H * W
    idx = np.arange(n, dtype=np.int64)
    passes = [idx & 0xFFFF, idx >> 16] if dt == "bf16" else [idx]
    for p in passes:
        announce(f"iota {dt}")
        if dt == "bf16":
            t = torch.from_numpy(p.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(p.astype(np.uint32).view(np.int32)).view(torch.float32)
        t = t.reshape(B, 4 * h * KD, H, W)
        packed = psa.psa_pack_qkv(t.to(dev), h, KD)
        assert np.array_equal(bits(packed), O.pack_qkv(bits(t), B, h, KD, H, W))
        want_packed = O.pack_qkv(bits(t), B, h, KD, H, W)
        merged = psa.psa_merge_attn(packed[2:].contiguous(), B, h, KD, H, W)
        assert np.array_equal(bits(merged), O.merge_attn(want_packed[2:], B, h, KD, H, W))


@pytest.mark.parametrize("name", ["psa_fwd_bf16_40x40_peaked", "psa_fwd_bf16_80x80"])
def test_full_size_bit_exact(name):
    """The two large maps, whole tensors, in the launch configuration the benchmark times."""
    dev = device()
    w = I.WORKLOADS[name]
    announce(f"layout full {name}")
    qkv = I.make_workload_qkv(w)
    packed = psa.psa_pack_qkv(qkv.to(dev), w.heads, w.key_dim)
    want = O.pack_qkv(bits(qkv), w.B, w.heads, w.key_dim, w.H, w.W)
    assert np.array_equal(bits(packed), want)
    v = psa.psa_extract_v(packed, w.B, w.heads, w.key_dim, w.H, w.W)
    assert np.array_equal(bits(v), O.extract_v(want, w.B, w.heads, w.key_dim, w.H, w.W))
    merged = psa.psa_merge_attn(packed[:2].contiguous(), w.B, w.heads, w.key_dim, w.H, w.W)
    assert np.array_equal(bits(merged), O.merge_attn(want[:2], w.B, w.heads, w.key_dim, w.H, w.W))


def test_stale_hip_error_is_not_reported_as_a_launch_failure():
    """A HIP error left on this thread by an earlier, unrelated call (here hipSetDevice on a
    device that does not exist) must not come back as an entry point's PSA_ERR_LAUNCH: the entry
    point clears it before its launches, which then succeed."""
    import ctypes
    dev = device()
    hip = ctypes.CDLL("libamdhip64.so")
    B, h, KD, H, W = 1, 2, 32, 4, 4
    qkv = I.make_qkv(B, h, KD, H, W, dtype="bf16", seed=5)
    x = qkv.to(dev)
    torch.cuda.synchronize()
    announce("psa_pack_qkv after a stale hipSetDevice(9999) error")
    assert hip.hipSetDevice(9999) != 0
    packed = psa.psa_pack_qkv(x, h, KD)
    torch.cuda.synchronize()
    assert np.array_equal(bits(packed), O.pack_qkv(bits(qkv), B, h, KD, H, W))


# The largest slabs: one (batch-head, slot) slab of key_dim 128 just under 2 GB (the LDS
# kernels, whose NCHW-side buffer stores take 32-bit offsets) and exactly 2 GB (the scalar
# kernel). (dtype, H, W)
LARGEST = [("f32", 8, 524287), ("f32", 2048, 2048), ("bf16", 8, 1048575), ("bf16", 2048, 4096)]


@pytest.mark.parametrize("case", LARGEST, ids=lambda c: "{}_{}x{}".format(*c))
def test_layout_largest_slab(case):
    """Pack, extract and merge on key_dim-128 maps whose slabs sit at the 2 GB edge, filled
    with random bit patterns on the GPU. The ops move each pixel's channels independently, so
    windows of 64 pixels (the first, one in the middle, the last) are checked against the
    oracle applied to the same windows of the inputs, bit for bit."""
    dev = device()
    dt, H, W = case
    B, h, KD = 1, 1, 128
    N = H * W
    announce(f"layout largest slab {dt} {H}x{W} key_dim {KD}")
    ity, fty = (torch.int32, torch.float32) if dt == "f32" else (torch.int16, torch.bfloat16)
    lo, hi = (-2 ** 31, 2 ** 31 - 1) if dt == "f32" else (-2 ** 15, 2 ** 15 - 1)
    g = torch.Generator(device=dev)
    g.manual_seed(777)
    qkv = torch.randint(lo, hi, (B, 4 * h * KD, H, W), generator=g, dtype=ity, device=dev).view(fty)
    packed = psa.psa_pack_qkv(qkv, h, KD)
    v = psa.psa_extract_v(packed, B, h, KD, H, W)
    del qkv
    o2 = torch.randint(lo, hi, (2, B * h, N, KD), generator=g, dtype=ity, device=dev).view(fty)
    merged = psa.psa_merge_attn(o2, B, h, KD, H, W)
    torch.cuda.synchronize()
    g.manual_seed(777)   # the same qkv bits again, for the windows
    qkv = torch.randint(lo, hi, (B, 4 * h * KD, H, W), generator=g, dtype=ity, device=dev).view(fty)
    w = 64
    for n0 in (0, (N // 2) // w * w, N - w):
        sl = slice(n0, n0 + w)
        q_win = bits(qkv.reshape(B, 4 * h * KD, N)[:, :, sl]).reshape(B, 4 * h * KD, 1, w)
        want_p = O.pack_qkv(q_win, B, h, KD, 1, w)
        assert np.array_equal(bits(packed[:, :, sl, :]), want_p), f"pack differs at pixels {n0}.."
        got_v = bits(v.reshape(B, 2 * h * KD, N)[:, :, sl]).reshape(B, 2 * h * KD, 1, w)
        assert np.array_equal(got_v, O.extract_v(want_p, B, h, KD, 1, w)), f"extract differs at pixels {n0}.."
        got_m = bits(merged.reshape(B, 2 * h * KD, N)[:, :, sl]).reshape(B, 2 * h * KD, 1, w)
        want_m = O.merge_attn(bits(o2[:, :, sl, :]), B, h, KD, 1, w)
        assert np.array_equal(got_m, want_m), f"merge differs at pixels {n0}.."
