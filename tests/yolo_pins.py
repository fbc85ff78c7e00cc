"""Checks that pin the detect-decode and CIoU oracle to facts other than itself: hand-worked
examples (tests/golden/), closed forms, invariants, finite differences and torch autograd.
Each check takes the oracle function(s) as arguments, so planted mistakes can be run through
the same checks."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def check_decode(detect_decode):
    ex = json.load(open(os.path.join(GOLDEN, "detect_decode_worked.json")))
    got = detect_decode(np.array(ex["boxes_ltrb"], dtype=np.float64).reshape(1, 4, 1),
                        np.array([ex["anchor_x"]]), np.array([ex["anchor_y"]]), np.array([ex["stride"]]))
    assert np.allclose(got[0, :, 0], ex["expected_cxcywh"], atol=1e-12), "worked example"
    rng = np.random.default_rng(3)
    B, A = 2, 50
    ax, ay = rng.uniform(0, 80, A), rng.uniform(0, 80, A)
    s = rng.choice([8.0, 16.0, 32.0], A)
    d = rng.uniform(0, 10, (B, 4, A))
    out = detect_decode(d, ax, ay, s)
    assert out.shape == (B, 4, A), "shape"
    # zero distances: a point box at the anchor, in pixels
    z = detect_decode(np.zeros((B, 4, A)), ax, ay, s)
    assert np.allclose(z[:, 0], ax * s) and np.allclose(z[:, 1], ay * s) and np.allclose(z[:, 2:], 0), "zero box"
    # width and height are the summed distances; the corners come back exactly
    l, t, r, b = d[:, 0], d[:, 1], d[:, 2], d[:, 3]
    assert np.allclose(out[:, 2], (l + r) * s) and np.allclose(out[:, 3], (t + b) * s), "w, h"
    assert np.allclose(out[:, 0] - out[:, 2] / 2, (ax - l) * s), "left edge"
    assert np.allclose(out[:, 1] + out[:, 3] / 2, (ay + b) * s), "bottom edge"
    # symmetric distances keep the centre on the anchor
    sym = d.copy(); sym[:, 2] = sym[:, 0]; sym[:, 3] = sym[:, 1]
    c = detect_decode(sym, ax, ay, s)
    assert np.allclose(c[:, 0], ax * s) and np.allclose(c[:, 1], ay * s), "symmetric box centre"


def check_ciou_forward(ciou_forward):
    ex = json.load(open(os.path.join(GOLDEN, "ciou_worked.json")))
    for case in ex["cases"]:
        p = np.array(case["pred_cxcywh"], dtype=np.float64).reshape(4, 1)
        g = np.array(case["target_cxcywh"], dtype=np.float64).reshape(4, 1)
        loss, iou, v, alpha = ciou_forward(p, g)
        assert abs(iou[0] - case["iou"]) < 1e-6, "worked example: iou"
        assert abs(v[0] - case["v"]) < 1e-6, "worked example: v"
        assert abs(loss[0] - case["loss"]) < 1e-6, "worked example: loss"
    rng = np.random.default_rng(5)
    N = 200
    p = np.stack([rng.uniform(0, 100, N), rng.uniform(0, 100, N), rng.uniform(1, 30, N), rng.uniform(1, 30, N)])
    g = np.stack([rng.uniform(0, 100, N), rng.uniform(0, 100, N), rng.uniform(1, 30, N), rng.uniform(1, 30, N)])
    # identical boxes: IoU 1, v 0, loss 0
    loss, iou, v, alpha = ciou_forward(p, p)
    assert np.allclose(iou, 1, atol=1e-6) and np.allclose(v, 0) and np.allclose(loss, 0, atol=1e-6), "identical"
    # far apart: IoU 0 and loss = 1 + rho^2/c^2 + alpha v with alpha = v / (1 + v)
    far = g.copy(); far[0] += 1000.0
    loss, iou, v, alpha = ciou_forward(p, far)
    assert np.allclose(iou, 0) and np.all(loss > 1), "disjoint"
    assert np.allclose(alpha, v / (1 + v), atol=1e-6), "disjoint alpha"
    # scale invariance of every term (a common factor on all coordinates)
    l1, i1, v1, _ = ciou_forward(p, g)
    l2, i2, v2, _ = ciou_forward(3.0 * p, 3.0 * g)
    assert np.allclose(l1, l2, atol=1e-6) and np.allclose(i1, i2, atol=1e-6) and np.allclose(v1, v2, atol=1e-6), "scale"
    # symmetry of IoU and v in the two boxes
    _, i3, v3, _ = ciou_forward(g, p)
    assert np.allclose(i1, i3) and np.allclose(v1, v3, atol=1e-9), "symmetry"
    assert np.all((i1 >= 0) & (i1 <= 1)) and np.all(v1 >= 0) and np.all(l1 >= 0) and np.all(l1 <= 3), "ranges"


def _ciou_torch(p, g, alpha):
    """The same loss written with torch ops (alpha given, held constant)."""
    eps = 1e-7
    px1, py1, px2, py2 = p[0] - p[2] / 2, p[1] - p[3] / 2, p[0] + p[2] / 2, p[1] + p[3] / 2
    gx1, gy1, gx2, gy2 = g[0] - g[2] / 2, g[1] - g[3] / 2, g[0] + g[2] / 2, g[1] + g[3] / 2
    inter = (torch.minimum(px2, gx2) - torch.maximum(px1, gx1)).clamp(min=0) * \
            (torch.minimum(py2, gy2) - torch.maximum(py1, gy1)).clamp(min=0)
    iou = inter / (p[2] * p[3] + g[2] * g[3] - inter + eps)
    c2 = (torch.maximum(px2, gx2) - torch.minimum(px1, gx1)) ** 2 + \
         (torch.maximum(py2, gy2) - torch.minimum(py1, gy1)) ** 2 + eps
    rho2 = (p[0] - g[0]) ** 2 + (p[1] - g[1]) ** 2
    v = (4 / math.pi ** 2) * (torch.atan(g[2] / (g[3] + eps)) - torch.atan(p[2] / (p[3] + eps))) ** 2
    return 1 - (iou - rho2 / c2 - alpha * v)


def check_ciou_backward(ciou_backward, ciou_forward):
    rng = np.random.default_rng(9)
    N = 40
    p = np.stack([rng.uniform(0, 20, N), rng.uniform(0, 20, N), rng.uniform(2, 10, N), rng.uniform(2, 10, N)])
    g = np.stack([rng.uniform(0, 20, N), rng.uniform(0, 20, N), rng.uniform(2, 10, N), rng.uniform(2, 10, N)])
    dloss = rng.normal(size=N)
    _, _, _, alpha = ciou_forward(p, g)
    grad = ciou_backward(p, g, alpha, dloss)
    assert grad.shape == p.shape, "gradient shape"
    # torch float64 autograd with alpha held constant
    tp = torch.tensor(p, requires_grad=True)
    (_ciou_torch(tp, torch.tensor(g), torch.tensor(alpha)) * torch.tensor(dloss)).sum().backward()
    assert np.allclose(grad, tp.grad.numpy(), atol=1e-10, rtol=0), "CIoU backward disagrees with torch autograd"
    # central finite differences of sum(dloss * loss), alpha held constant
    def loss_fixed_alpha(pp):
        l, iou, v, _ = ciou_forward(pp, g)
        # replace the forward's alpha v term by the fixed alpha's
        _, _, v_now, a_now = ciou_forward(pp, g)
        return float((dloss * (l - a_now * v_now + alpha * v_now)).sum())
    eps = 1e-6
    num = np.zeros_like(p)
    for idx in np.ndindex(*p.shape):
        old = p[idx]
        p[idx] = old + eps; lp = loss_fixed_alpha(p)
        p[idx] = old - eps; lm = loss_fixed_alpha(p)
        p[idx] = old
        num[idx] = (lp - lm) / (2 * eps)
    assert np.allclose(grad, num, atol=1e-6, rtol=1e-5), "CIoU backward disagrees with finite differences"
