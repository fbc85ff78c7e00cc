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
