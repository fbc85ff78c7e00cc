"""The detect-decode and CIoU oracle against its pins, and the pins against planted mistakes (CPU)."""
import math

import numpy as np
import pytest

from oracle import yolo_oracle as Y
from tests import yolo_pins as pins


def test_decode_pins():
    pins.check_decode(Y.detect_decode)


def test_ciou_forward_pins():
    pins.check_ciou_forward(Y.ciou_forward)


def test_ciou_backward_pins():
    pins.check_ciou_backward(Y.ciou_backward, Y.ciou_forward)


def _decode_variant(mode):
    def detect_decode(boxes, ax, ay, s):
        x = np.asarray(boxes, dtype=np.float64)
        l, t, r, b = x[:, 0], x[:, 1], x[:, 2], x[:, 3]
        if mode == "lr_swapped":
            l, r = r, l
        x1, y1, x2, y2 = ax - l, ay - t, ax + r, ay + b
        k = 1.0 if mode == "no_stride" else s
        if mode == "xyxy":
            return np.stack([x1 * k, y1 * k, x2 * k, y2 * k], axis=1)
        return np.stack([(x1 + x2) / 2 * k, (y1 + y2) / 2 * k, (x2 - x1) * k, (y2 - y1) * k], axis=1)
    return detect_decode


@pytest.mark.parametrize("mode", ["lr_swapped", "no_stride", "xyxy"])
def test_decode_mutants_are_caught(mode):
    with pytest.raises(AssertionError):
        pins.check_decode(_decode_variant(mode))


def _ciou_fwd_variant(mode):
    def ciou_forward(pred, target):
        loss, iou, v, alpha = Y.ciou_forward(pred, target)
        p, g = np.asarray(pred, dtype=np.float64), np.asarray(target, dtype=np.float64)
        if mode == "no_rho":
            cw = np.maximum(p[0] + p[2] / 2, g[0] + g[2] / 2) - np.minimum(p[0] - p[2] / 2, g[0] - g[2] / 2)
            ch = np.maximum(p[1] + p[3] / 2, g[1] + g[3] / 2) - np.minimum(p[1] - p[3] / 2, g[1] - g[3] / 2)
            loss = loss - ((p[0] - g[0]) ** 2 + (p[1] - g[1]) ** 2) / (cw ** 2 + ch ** 2 + 1e-7)
        if mode == "no_aspect":
            loss = loss - alpha * v
        return loss, iou, v, alpha
    return ciou_forward


@pytest.mark.parametrize("mode", ["no_rho", "no_aspect"])
def test_ciou_forward_mutants_are_caught(mode):
    with pytest.raises(AssertionError):
        pins.check_ciou_forward(_ciou_fwd_variant(mode))


def _ciou_bwd_variant(mode):
    def ciou_backward(pred, target, alpha, dloss):
        g = Y.ciou_backward(pred, target, alpha, dloss)
        if mode == "w_h_swapped":
            g = g[[0, 1, 3, 2]]
        if mode == "no_aspect_grad":
            g = Y.ciou_backward(pred, target, np.zeros_like(alpha), dloss)
        if mode == "sign":
            g = -g
        return g
    return ciou_backward


@pytest.mark.parametrize("mode", ["w_h_swapped", "no_aspect_grad", "sign"])
def test_ciou_backward_mutants_are_caught(mode):
    with pytest.raises(AssertionError):
        pins.check_ciou_backward(_ciou_bwd_variant(mode), Y.ciou_forward)
