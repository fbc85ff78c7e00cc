"""Seeded synthetic inputs for the detect-decode and CIoU-loss kernels.

Shared by the tests and the benchmark. It only draws random numbers and lays
out the anchor grid (the precomputed per-anchor state the decode consumes); it
contains none of the decode or loss arithmetic. There is no dataset behind
these boxes: the shapes follow a YOLO head on 640x640 images.

Recipe (numpy PCG64, one generator per call, seeded explicitly; float32 draws):
  * anchor grid of an image of IMG_H x IMG_W pixels at strides 8, 16, 32: for
    each stride s the grid has (IMG_H / s) x (IMG_W / s) cells in row-major
    order, anchor_x = x + 0.5, anchor_y = y + 0.5 (cell centres in grid units)
    and strides = s; the three levels are concatenated, finest first. A 640x640
    image gives A = 6400 + 1600 + 400 = 8400 anchors;
  * LTRB box distances [B, 4, A]: U[0, 16) grid cells (the range of a
    16-bin distribution-focal head's expected distance);
  * CIoU target boxes [4, N] (cx, cy, w, h in pixels): centres U[0, 640),
    sides exp(U[log 8, log 320)); predicted boxes: the target moved by
    N(0, (0.15 w)^2) and N(0, (0.15 h)^2) with sides scaled by exp(N(0, 0.25^2)),
    except a fraction `far` of them drawn independently like the targets (mostly
    disjoint pairs); the upstream gradient dloss [N] is U[0.5, 1.5).
"""
from __future__ import annotations

import numpy as np
import torch

STRIDES = (8, 16, 32)


def anchor_grid(img_h: int = 640, img_w: int = 640, strides=STRIDES):
    """``(anchor_x, anchor_y, strides)``, each a float32 CPU tensor of shape ``[A]``."""
    xs, ys, ss = [], [], []
    for s in strides:
        gh, gw = img_h // s, img_w // s
        y, x = np.meshgrid(np.arange(gh, dtype=np.float32), np.arange(gw, dtype=np.float32),
                           indexing="ij")
        xs.append(x.reshape(-1) + 0.5)
        ys.append(y.reshape(-1) + 0.5)
        ss.append(np.full(gh * gw, s, dtype=np.float32))
    return tuple(torch.from_numpy(np.ascontiguousarray(np.concatenate(t))) for t in (xs, ys, ss))


def ltrb_boxes(B: int, A: int, *, dtype=torch.float32, seed: int = 0) -> torch.Tensor:
    """Raw LTRB distances ``[B, 4, A]`` in grid units (CPU)."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(0.0, 16.0, size=(B, 4, A)).astype(np.float32)
    return torch.from_numpy(x).to(dtype).contiguous()


def _boxes(rng, N):
    c = rng.uniform(0.0, 640.0, size=(2, N))
    s = np.exp(rng.uniform(np.log(8.0), np.log(320.0), size=(2, N)))
    return np.concatenate([c, s]).astype(np.float32)


def ciou_boxes(N: int, *, far: float = 0.1, seed: int = 0):
    """``(pred, target, dloss)``: ``[4, N]``, ``[4, N]``, ``[N]`` float32 CPU tensors."""
    rng = np.random.default_rng(seed)
    tgt = _boxes(rng, N)
    pred = np.empty_like(tgt)
    pred[0] = tgt[0] + rng.normal(0.0, 1.0, N) * 0.15 * tgt[2]
    pred[1] = tgt[1] + rng.normal(0.0, 1.0, N) * 0.15 * tgt[3]
    pred[2] = tgt[2] * np.exp(rng.normal(0.0, 0.25, N))
    pred[3] = tgt[3] * np.exp(rng.normal(0.0, 0.25, N))
    other = _boxes(rng, N)
    pick = rng.uniform(size=N) < far
    pred[:, pick] = other[:, pick]
    dloss = rng.uniform(0.5, 1.5, size=N).astype(np.float32)
    return tuple(torch.from_numpy(np.ascontiguousarray(t.astype(np.float32))) for t in (pred, tgt, dloss))
