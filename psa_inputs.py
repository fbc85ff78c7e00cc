"""Seeded synthetic inputs for the PSA attention path.

This module is shared by the tests, the benchmark and the CPU checker. It
only draws random numbers and rounds them to the storage dtype; it contains
none of the arithmetic of the PSA path itself (no packing, no softmax, no
merge). Every workload is synthetic: there is no dataset behind these maps.

Recipe (one numpy PCG64 generator per tensor set, seeded explicitly):
  * draws are float32, generated in C order over the whole tensor;
  * bf16 tensors are the float32 draw rounded to nearest-even by torch on the
    CPU (``Tensor.to(torch.bfloat16)``);
  * the "peaked" 40x40 workload multiplies the query channels of the float32
    draw by 3 before rounding, so that softmax rows are sharper.

The query channels are the first KEY_DIM channels of each head's
``[Q | K | V_lo | V_hi]`` group (vision-rs book, "Custom Kernels",
section "Position-Sensitive Attention (PSA)", description of PsaPackQkv).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class PsaWorkload:
    """One synthetic PSA feature-map workload (forward) or FA2 backward set."""
    name: str
    B: int
    heads: int
    key_dim: int
    H: int
    W: int
    dtype: str          # "f32" or "bf16"
    dist: str           # "uniform" (U(-1,1)) or "normal" (N(0,1))
    q_scale: float      # factor applied to the query channels before rounding
    seed: int
    kind: str = "fwd"   # "fwd" (PSA forward on an NCHW map) or "bwd" (FA2 backward)

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def BH(self) -> int:
        return self.B * self.heads

    @property
    def qkv_channels(self) -> int:
        return 4 * self.heads * self.key_dim

    @property
    def out_channels(self) -> int:
        return 2 * self.heads * self.key_dim


# The five workloads the path is measured and checked on. The 20x20, 40x40 and
# 80x80 maps are the stride-32/16/8 feature maps of a 640x640 image.
WORKLOADS = {
    "psa_fwd_f32_tiny_8x8": PsaWorkload(
        "psa_fwd_f32_tiny_8x8", B=1, heads=1, key_dim=16, H=8, W=8,
        dtype="f32", dist="uniform", q_scale=1.0, seed=1000),
    "psa_fwd_bf16_20x20": PsaWorkload(
        "psa_fwd_bf16_20x20", B=8, heads=4, key_dim=32, H=20, W=20,
        dtype="bf16", dist="normal", q_scale=1.0, seed=1001),
    "psa_fwd_bf16_40x40_peaked": PsaWorkload(
        "psa_fwd_bf16_40x40_peaked", B=32, heads=8, key_dim=32, H=40, W=40,
        dtype="bf16", dist="normal", q_scale=3.0, seed=1002),
    "psa_fwd_bf16_80x80": PsaWorkload(
        "psa_fwd_bf16_80x80", B=4, heads=8, key_dim=64, H=80, W=80,
        dtype="bf16", dist="normal", q_scale=1.0, seed=1003),
    "fa2_bwd_bf16_40x40": PsaWorkload(
        "fa2_bwd_bf16_40x40", B=32, heads=8, key_dim=32, H=40, W=40,
        dtype="bf16", dist="normal", q_scale=1.0, seed=1004, kind="bwd"),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(size=shape, dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def _store(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(TORCH_DTYPE[dtype]).contiguous()


def make_qkv(B: int, heads: int, key_dim: int, H: int, W: int, *, dtype: str = "bf16",
             dist: str = "normal", q_scale: float = 1.0, seed: int = 0) -> torch.Tensor:
    """NCHW QKV-conv output ``[B, 4*heads*key_dim, H, W]`` on the CPU."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (B, 4 * heads * key_dim, H, W), dist)
    if q_scale != 1.0:
        # Query channels: the first key_dim channels of each head's group of 4*key_dim.
        grouped = x.reshape(B, heads, 4 * key_dim, H, W)
        grouped[:, :, :key_dim] *= np.float32(q_scale)
    return _store(x, dtype)


def make_workload_qkv(w: PsaWorkload) -> torch.Tensor:
    return make_qkv(w.B, w.heads, w.key_dim, w.H, w.W, dtype=w.dtype, dist=w.dist,
                    q_scale=w.q_scale, seed=w.seed)


def make_attention_inputs(BH: int, n_q: int, n_k: int, head_dim: int, *, dtype: str = "bf16",
                          dist: str = "normal", seed: int = 0, with_dout: bool = False,
                          head_dim_v: int | None = None):
    """Q ``[BH,n_q,D]``, K ``[BH,n_k,D]``, V ``[BH,n_k,Dv]`` (and dO ``[BH,n_q,Dv]``), drawn in that order."""
    dv = head_dim if head_dim_v is None else head_dim_v
    rng = np.random.default_rng(seed)
    q = _store(_draw(rng, (BH, n_q, head_dim), dist), dtype)
    k = _store(_draw(rng, (BH, n_k, head_dim), dist), dtype)
    v = _store(_draw(rng, (BH, n_k, dv), dist), dtype)
    if not with_dout:
        return q, k, v
    do = _store(_draw(rng, (BH, n_q, dv), dist), dtype)
    return q, k, v, do


def make_workload_bwd(w: PsaWorkload):
    """Q, K, V, dO for the FA2 backward workload (one FA2 call, head_dim = key_dim)."""
    return make_attention_inputs(w.BH, w.N, w.N, w.key_dim, dtype=w.dtype, dist=w.dist,
                                 seed=w.seed, with_dout=True)


# Score ramps: query and key rows built so that the dot product q_n . k_m grows
# (even n) or falls (odd n) linearly along the key index m, by score_step per key,
# plus a little N(0, noise^2) on every element (no exact ties). With u the unit
# vector of ones / sqrt(dim): q_n = 8 * (+-1) * u + noise, k_m = (m * score_step / 8) * u
# + noise. V is N(0, 1); dO is N(0, dout_scale^2) (the rising queries all put their
# weight on the last keys, so dK and dV sum many dO rows).
_RAMP_Q = 8.0


def _ramp_qk(rng: np.random.Generator, lead, n_q: int, n_k: int, dim: int, score_step: float,
             noise: float):
    u = np.full(dim, 1.0 / np.sqrt(dim), dtype=np.float32)
    sign = np.where(np.arange(n_q) % 2 == 0, 1.0, -1.0).astype(np.float32)
    t = np.arange(n_k, dtype=np.float32) * np.float32(score_step / _RAMP_Q)
    q = np.float32(_RAMP_Q) * sign[:, None] * u[None, :] + np.float32(noise) * rng.standard_normal(
        tuple(lead) + (n_q, dim), dtype=np.float32)
    k = t[:, None] * u[None, :] + np.float32(noise) * rng.standard_normal(tuple(lead) + (n_k, dim), dtype=np.float32)
    return q, k


def make_ramp_attention_inputs(BH: int, n_q: int, n_k: int, head_dim: int, *, score_step: float,
                               seed: int = 0, noise: float = 0.05, with_dout: bool = False,
                               dout_scale: float = 0.25):
    """bf16 Q ``[BH,n_q,D]`` and K ``[BH,n_k,D]`` on a score ramp (see above), V ``[BH,n_k,D]``
    drawn N(0, 1) and dO ``[BH,n_q,D]`` N(0, dout_scale^2)."""
    rng = np.random.default_rng(seed)
    q, k = _ramp_qk(rng, (BH,), n_q, n_k, head_dim, score_step, noise)
    v = rng.standard_normal((BH, n_k, head_dim), dtype=np.float32)
    out = [_store(q, "bf16"), _store(k, "bf16"), _store(v, "bf16")]
    if with_dout:
        out.append(_store(np.float32(dout_scale) * rng.standard_normal((BH, n_q, head_dim), dtype=np.float32),
                          "bf16"))
    return tuple(out)


def make_ramp_qkv(B: int, heads: int, key_dim: int, H: int, W: int, *, score_step: float,
                  seed: int = 0, noise: float = 0.05) -> torch.Tensor:
    """bf16 NCHW QKV-conv output ``[B, 4*heads*key_dim, H, W]`` whose query and key channels
    (the first and second key_dim channels of each head's group) hold a score ramp over the
    pixel index; the V channels are N(0, 1)."""
    rng = np.random.default_rng(seed)
    N = H * W
    x = rng.standard_normal((B, heads, 4, key_dim, N), dtype=np.float32)
    q, k = _ramp_qk(rng, (B, heads), N, N, key_dim, score_step, noise)   # [B, heads, N, KD]
    x[:, :, 0] = np.swapaxes(q, -1, -2)
    x[:, :, 1] = np.swapaxes(k, -1, -2)
    return _store(x.reshape(B, 4 * heads * key_dim, H, W), "bf16")


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a stored f32/bf16 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """The stored bit patterns (uint16 for bf16, uint32 for f32) as numpy."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(f"unsupported dtype {t.dtype}")
