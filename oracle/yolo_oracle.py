"""Plain CPU oracle for the detect-decode and CIoU-loss kernels (float64, numpy).

TEST INFRASTRUCTURE ONLY, like psa_oracle: only the tests, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg may use it; it shares no code with the HIP
library, and the library never falls back to it.

What it follows: vision-rs book, "Custom Kernels", section "Detect-decode" (the
head's LTRB distances and an anchor grid computed beforehand, turned into
[cx, cy, w, h] boxes in one pass; the anchor grid is anchor_x, anchor_y and strides, one value per
anchor) and section "Loss kernels", ``ciou`` bullet (predicted and target
[4, N] XYWH boxes in, per-anchor loss plus the iou, v and alpha the backward
needs out). The teenygrad book, "Your Kernel as a Graph Op", shows the decode's
boxes as [B, 4, A] and its three per-anchor parameters.

Readings where the pages are silent (each is also listed in the design notes):
  * decode: distances and anchors are in grid units, the output in pixels:
    x1 = ax - l, y1 = ay - t, x2 = ax + r, y2 = ay + b, then
    [cx, cy, w, h] = [(x1 + x2) / 2, (y1 + y2) / 2, x2 - x1, y2 - y1] * stride;
    channel order of the predictions is (l, t, r, b);
  * CIoU is the complete-IoU of Zheng et al. (AAAI 2020): with IoU of the two
    boxes, rho^2 the squared distance of their centres, c^2 the squared diagonal
    of the smallest box enclosing both, v = (4 / pi^2)(atan(w_t / h_t) -
    atan(w_p / h_p))^2 and alpha = v / (1 - IoU + v): CIoU = IoU - rho^2 / c^2 -
    alpha v, and the loss is 1 - CIoU;
  * eps = 1e-7 guards the divisions: union + eps, c^2 + eps, heights + eps inside
    the arctangents, and alpha = v / (v - IoU + 1 + eps);
  * the backward gives the gradient with respect to the predicted boxes only
    (targets are data), with alpha held constant (the saved alpha is used as
    is, so no gradient flows through it).
"""
from __future__ import annotations

import math

import numpy as np

EPS = 1e-7


def detect_decode(boxes: np.ndarray, anchor_x: np.ndarray, anchor_y: np.ndarray,
                  strides: np.ndarray) -> np.ndarray:
    """``boxes [B, 4, A]`` LTRB (grid units) + anchors ``[A]`` -> ``[B, 4, A]`` cx, cy, w, h (pixels)."""
    x = np.asarray(boxes, dtype=np.float64)
    ax, ay, s = (np.asarray(t, dtype=np.float64) for t in (anchor_x, anchor_y, strides))
    l, t, r, b = x[:, 0], x[:, 1], x[:, 2], x[:, 3]
    x1, y1, x2, y2 = ax - l, ay - t, ax + r, ay + b
    return np.stack([(x1 + x2) / 2 * s, (y1 + y2) / 2 * s, (x2 - x1) * s, (y2 - y1) * s], axis=1)


def _corners(box):
    cx, cy, w, h = box
    return cx - w / 2, cy - h / 2, cx + w / 2, cy + h / 2


def ciou_forward(pred: np.ndarray, target: np.ndarray):
    """Per-anchor CIoU loss of ``[4, N]`` cx, cy, w, h boxes: returns ``(loss, iou, v, alpha)``."""
    p = np.asarray(pred, dtype=np.float64)
    g = np.asarray(target, dtype=np.float64)
    px1, py1, px2, py2 = _corners(p)
    gx1, gy1, gx2, gy2 = _corners(g)
    iw = np.clip(np.minimum(px2, gx2) - np.maximum(px1, gx1), 0.0, None)
    ih = np.clip(np.minimum(py2, gy2) - np.maximum(py1, gy1), 0.0, None)
    inter = iw * ih
    union = p[2] * p[3] + g[2] * g[3] - inter + EPS
    iou = inter / union
    cw = np.maximum(px2, gx2) - np.minimum(px1, gx1)
    ch = np.maximum(py2, gy2) - np.minimum(py1, gy1)
    c2 = cw ** 2 + ch ** 2 + EPS
    rho2 = (p[0] - g[0]) ** 2 + (p[1] - g[1]) ** 2
    v = (4.0 / math.pi ** 2) * (np.arctan(g[2] / (g[3] + EPS)) - np.arctan(p[2] / (p[3] + EPS))) ** 2
    alpha = v / (v - iou + 1.0 + EPS)
    loss = 1.0 - (iou - rho2 / c2 - alpha * v)
    return loss, iou, v, alpha


def ciou_backward(pred: np.ndarray, target: np.ndarray, alpha: np.ndarray, dloss: np.ndarray) -> np.ndarray:
    """Gradient ``[4, N]`` of sum(dloss * loss) with respect to ``pred`` (cx, cy, w, h), alpha held
    constant: the derivative of loss = 1 - IoU + rho^2/c^2 + alpha v, term by term."""
    p = np.asarray(pred, dtype=np.float64)
    g = np.asarray(target, dtype=np.float64)
    a = np.asarray(alpha, dtype=np.float64)
    dl = np.asarray(dloss, dtype=np.float64)
    cx, cy, w, h = p
    px1, py1, px2, py2 = _corners(p)
    gx1, gy1, gx2, gy2 = _corners(g)
    # d(corner)/d(cx, cy, w, h): x1 = cx - w/2, x2 = cx + w/2, y1 = cy - h/2, y2 = cy + h/2
    zero = np.zeros_like(cx)

    def grad_from_corners(dx1, dy1, dx2, dy2):
        return np.stack([dx1 + dx2, dy1 + dy2, (dx2 - dx1) / 2, (dy2 - dy1) / 2])

    # IoU = inter / union, inter = iw * ih, union = w h + w_g h_g - inter + eps
    ix1, ix2 = np.maximum(px1, gx1), np.minimum(px2, gx2)
    iy1, iy2 = np.maximum(py1, gy1), np.minimum(py2, gy2)
    iw_raw, ih_raw = ix2 - ix1, iy2 - iy1
    iw, ih = np.clip(iw_raw, 0.0, None), np.clip(ih_raw, 0.0, None)
    inter = iw * ih
    union = w * h + g[2] * g[3] - inter + EPS
    # d iw / d px1 = -1 if px1 > gx1 (and iw_raw > 0); d iw / d px2 = +1 if px2 < gx2
    on_w, on_h = iw_raw > 0, ih_raw > 0
    diw_dx1 = np.where(on_w & (px1 > gx1), -1.0, 0.0)
    diw_dx2 = np.where(on_w & (px2 < gx2), 1.0, 0.0)
    dih_dy1 = np.where(on_h & (py1 > gy1), -1.0, 0.0)
    dih_dy2 = np.where(on_h & (py2 < gy2), 1.0, 0.0)
    dinter = grad_from_corners(diw_dx1 * ih, dih_dy1 * iw, diw_dx2 * ih, dih_dy2 * iw)
    darea = np.stack([zero, zero, h, w])                  # d(w h) / d(cx, cy, w, h)
    dunion = darea - dinter
    diou = (dinter * union - inter * dunion) / union ** 2
    # rho^2 / c^2
    rho2 = (cx - g[0]) ** 2 + (cy - g[1]) ** 2
    drho2 = np.stack([2 * (cx - g[0]), 2 * (cy - g[1]), zero, zero])
    ex1, ex2 = np.minimum(px1, gx1), np.maximum(px2, gx2)
    ey1, ey2 = np.minimum(py1, gy1), np.maximum(py2, gy2)
    cw, ch = ex2 - ex1, ey2 - ey1
    c2 = cw ** 2 + ch ** 2 + EPS
    dcw = grad_from_corners(np.where(px1 < gx1, -1.0, 0.0), zero, np.where(px2 > gx2, 1.0, 0.0), zero)
    dch = grad_from_corners(zero, np.where(py1 < gy1, -1.0, 0.0), zero, np.where(py2 > gy2, 1.0, 0.0))
    dc2 = 2 * cw * dcw + 2 * ch * dch
    dratio = (drho2 * c2 - rho2 * dc2) / c2 ** 2
    # v = k (atan(w_g/(h_g+eps)) - atan(w/(h+eps)))^2, d/dw and d/dh of atan(w/(h+eps))
    k = 4.0 / math.pi ** 2
    diff = np.arctan(g[2] / (g[3] + EPS)) - np.arctan(w / (h + EPS))
    he = h + EPS
    datan = np.stack([zero, zero, he / (he ** 2 + w ** 2), -w / (he ** 2 + w ** 2)])
    dv = -2 * k * diff * datan
    return dl * (-diou + dratio + a * dv)
