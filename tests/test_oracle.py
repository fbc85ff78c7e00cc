"""The CPU oracle against its pins, and the pins against planted mistakes (CPU only)."""
import numpy as np
import pytest

from oracle import psa_oracle as O
from tests import oracle_pins as pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------ the oracle passes

def test_pack_pins():
    pins.check_pack(O.pack_qkv)


def test_extract_pins():
    pins.check_extract(O.pack_qkv, O.extract_v)


def test_merge_pins():
    pins.check_merge(O.merge_attn)


def test_attention_pins():
    pins.check_attention(O.attention)


def test_psa_forward_golden():
    pins.check_psa_golden(O.psa_forward, O.pack_qkv)


def test_attention_bwd_pins():
    pins.check_attention_bwd(O.attention_bwd, O.attention)


def test_layout_on_bits():
    """The layout functions move stored bit patterns unchanged (NaN payloads included)."""
    B, h, KD, H, W = 1, 2, 16, 3, 5
    bits = np.random.default_rng(0).integers(0, 2**16, size=(B, 4 * h * KD, H, W)).astype(np.uint16)
    bits.reshape(-1)[:5] = [0x7FC1, 0xFFFF, 0x7F80, 0x8000, 0x0001]
    packed = O.pack_qkv(bits, B, h, KD, H, W)
    assert packed.dtype == np.uint16
    assert np.array_equal(np.sort(packed.reshape(-1)), np.sort(bits.reshape(-1)))
    v = O.extract_v(packed, B, h, KD, H, W)
    assert np.array_equal(v, bits.reshape(B, h, 4, KD, H, W)[:, :, 2:].reshape(B, 2 * h * KD, H, W))


# ------------------------------------------- planted mistakes fail at least one pin

def _pack_variant(mode):
    def pack(qkv, B, heads, key_dim, H, W):
        KD, N, BH, C = key_dim, H * W, B * heads, 4 * heads * key_dim
        flat = np.asarray(qkv).reshape(-1)
        bh, n, d = np.ix_(np.arange(BH), np.arange(N), np.arange(KD))
        b, i = bh // heads, bh % heads
        if mode == "head_major_bh":
            b, i = bh % B, bh // B
        out = np.empty((4, BH, N, KD), dtype=flat.dtype)
        for s in range(4):
            if mode == "section_major":
                ch = s * heads * KD + i * KD + d
            elif mode == "slot_d_swapped":
                ch = i * 4 * KD + d * 4 + s
            else:
                ch = i * 4 * KD + s * KD + d
            nn = n
            if mode == "xy_swapped":
                nn = (n % W) * H + n // W
            out[s] = flat[(b * C + ch) * N + nn]
        return out
    return pack


@pytest.mark.parametrize("mode", ["head_major_bh", "section_major", "slot_d_swapped", "xy_swapped"])
def test_pack_mutants_are_caught(mode):
    with pytest.raises(AssertionError):
        pins.check_pack(_pack_variant(mode))


def test_extract_mutant_halves_swapped_is_caught():
    def extract(packed, B, heads, key_dim, H, W):
        p = np.asarray(packed).copy()
        p[[2, 3]] = p[[3, 2]]
        return O.extract_v(p, B, heads, key_dim, H, W)
    with pytest.raises(AssertionError):
        pins.check_extract(O.pack_qkv, extract)


def test_merge_mutant_halves_swapped_is_caught():
    def merge(o2, B, heads, key_dim, H, W):
        return O.merge_attn(np.asarray(o2)[::-1].copy(), B, heads, key_dim, H, W)
    with pytest.raises(AssertionError):
        pins.check_merge(merge)


def _attention_variant(mode):
    def attention(q, k, v, scale):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        BH, n_q, _ = q.shape
        o = np.empty((BH, n_q, v.shape[2])); lse = np.empty((BH, n_q))
        for bh in range(BH):
            s = (1.0 if mode == "no_scale" else scale) * (q[bh] @ k[bh].T)
            m = s.max(axis=1, keepdims=True)
            if mode == "no_max":
                m = np.zeros_like(m)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            zo = e.sum(axis=0, keepdims=True) if mode == "wrong_axis" else z
            o[bh] = (e / zo) @ v[bh]
            lse[bh] = (np.log(z) if mode == "lse_drops_max" else m + np.log(z))[:, 0]
        return o, lse
    return attention


@pytest.mark.parametrize("mode", ["no_scale", "no_max", "wrong_axis", "lse_drops_max"])
def test_attention_mutants_are_caught(mode):
    with pytest.raises(AssertionError):
        pins.check_attention(_attention_variant(mode))


def _bwd_variant(mode):
    def attention_bwd(q, k, v, dout, scale):
        o, lse = O.attention(q, k, v, scale)
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        for bh in range(q.shape[0]):
            p = np.exp(scale * (q[bh] @ k[bh].T) - lse[bh][:, None])
            dv[bh] = p.T @ dout[bh]
            dp = dout[bh] @ v[bh].T
            delta = (dout[bh] * o[bh]).sum(axis=1)
            if mode == "no_delta":
                delta = 0 * delta
            ds = p * (dp - delta[:, None]) if mode != "sign" else p * (delta[:, None] - dp)
            dq[bh] = scale * (ds @ k[bh])
            dk[bh] = (1.0 if mode == "dk_no_scale" else scale) * (ds.T @ q[bh])
            if mode == "dv_from_ds":
                dv[bh] = ds.T @ dout[bh]
        return dq, dk, dv
    return attention_bwd


@pytest.mark.parametrize("mode", ["no_delta", "sign", "dk_no_scale", "dv_from_ds"])
def test_bwd_mutants_are_caught(mode):
    with pytest.raises(AssertionError):
        pins.check_attention_bwd(_bwd_variant(mode), O.attention)


def test_golden_catches_section_major_pack():
    def psa_forward(qkv, B, heads, key_dim, H, W, scale=None):
        s = O.default_scale(key_dim) if scale is None else scale
        packed = _pack_variant("section_major")(np.asarray(qkv, dtype=np.float64), B, heads, key_dim, H, W)
        lo, lse = O.attention(packed[0], packed[1], packed[2], s)
        hi, _ = O.attention(packed[0], packed[1], packed[3], s)
        return (O.merge_attn(np.stack([lo, hi]), B, heads, key_dim, H, W),
                O.extract_v(packed, B, heads, key_dim, H, W), lse)
    with pytest.raises(AssertionError):
        pins.check_psa_golden(psa_forward, _pack_variant("section_major"))


def test_psa_backward_pins():
    pins.check_psa_backward(O.psa_backward, O.psa_forward)


def test_layout_inverses():
    """split_attn undoes merge_attn and unpack_qkv undoes pack_qkv (the adjoints of
    permutations are their inverses), also on raw bits."""
    B, h, KD, H, W = 2, 3, 4, 3, 5
    rng = np.random.default_rng(3)
    x = rng.integers(0, 2**16, size=(B, 4 * h * KD, H, W)).astype(np.uint16)
    assert np.array_equal(O.unpack_qkv(O.pack_qkv(x, B, h, KD, H, W), B, h, KD, H, W), x)
    o = rng.integers(0, 2**16, size=(B, 2 * h * KD, H, W)).astype(np.uint16)
    assert np.array_equal(O.merge_attn(O.split_attn(o, B, h, KD, H, W), B, h, KD, H, W), o)
    o2 = rng.integers(0, 2**16, size=(2, B * h, H * W, KD)).astype(np.uint16)
    assert np.array_equal(O.split_attn(O.merge_attn(o2, B, h, KD, H, W), B, h, KD, H, W), o2)


def _psa_bwd_variant(mode):
    def psa_backward(qkv, dout, dv_res, B, heads, key_dim, H, W, scale=None):
        s = O.default_scale(key_dim) if scale is None else scale
        packed = O.pack_qkv(np.asarray(qkv, dtype=np.float64), B, heads, key_dim, H, W)
        do2 = O.split_attn(np.asarray(dout, dtype=np.float64), B, heads, key_dim, H, W)
        if mode == "halves_swapped":
            do2 = do2[::-1]
        dq0, dk0, dv0 = O.attention_bwd(packed[0], packed[1], packed[2], do2[0], s)
        dq1, dk1, dv1 = O.attention_bwd(packed[0], packed[1], packed[3], do2[1], s)
        dq = dq0 if mode == "dq_lo_only" else dq0 + dq1
        dk = dk1 if mode == "dk_hi_only" else dk0 + dk1
        dp = np.stack([dq, dk, dv0, dv1])
        if dv_res is not None and mode != "no_vres":
            dp[2:] += O.split_attn(np.asarray(dv_res, dtype=np.float64), B, heads, key_dim, H, W)
        return O.unpack_qkv(dp, B, heads, key_dim, H, W)
    return psa_backward


@pytest.mark.parametrize("mode", ["halves_swapped", "dq_lo_only", "dk_hi_only", "no_vres"])
def test_psa_backward_mutants_are_caught(mode):
    with pytest.raises(AssertionError):
        pins.check_psa_backward(_psa_bwd_variant(mode), O.psa_forward)
