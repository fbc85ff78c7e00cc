"""Detect-decode and CIoU loss (forward, backward) through the C ABI against the float64 oracle.

Tolerances (derived from float32 arithmetic, u = 2^-24):
  * decode: x1 = ax - l and x2 = ax + r and their sum or difference are each
    rounded once (error <= u times the magnitude), the factor 1/2 and the
    strides (powers of two) are exact, so |err| <= 3u (|ax| + |l| + |r|) s per
    x output (likewise y); bf16 results add one final rounding to 8 significant
    bits, at most 2^-8 |value| (the unit roundoff of bf16).
  * CIoU: corners carry an error of u M (M the largest coordinate magnitude),
    so the overlap and the enclosing box are off by about 2 u M per side; over
    the smallest side s_min this is a relative error of 2 u M / s_min, which
    the quotients (IoU, rho^2/c^2, alpha) pass on with a few more roundings and
    the float32 arctangent (a few ulp). Tolerance: 32 u M / s_min + 1e-6.
    Gradient terms are products of O(1/s_min) factors with that relative
    error: |err| <= |dloss| (64 u M / s_min^2 + 1e-5 |grad|).
  * Where a box edge of the prediction and of the target lie within 1e-3 pixel
    of each other, the loss is not differentiable and float32 and float64 may
    take different one-sided derivatives: such anchors (a tiny fraction of the
    random pairs) are left out of the gradient comparison, and their count is
    checked to stay small.
"""
import numpy as np
import pytest
import torch

import vision_transformer_attention_psapackqkv_amd as psa
import yolo_inputs as yi
from oracle import yolo_oracle as Y
from tests.gpu_helpers import announce, device, to_f64

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _decode_case(B, A, dtype, seed, grid=None):
    dev = device()
    if grid is None:   # the 640x640 grid, repeated cyclically if A > 8400
        idx = torch.arange(A) % 8400
        ax, ay, st = (t[idx].contiguous() for t in yi.anchor_grid())
    else:
        ax, ay, st = grid
    boxes = yi.ltrb_boxes(B, A, dtype=dtype, seed=seed)
    announce(f"detect_decode B={B} A={A} dtype={dtype} seed={seed}")
    out = psa.detect_decode(boxes.to(dev), ax.to(dev), ay.to(dev), st.to(dev))
    torch.cuda.synchronize()
    assert out.dtype == dtype and out.shape == (B, 4, A)
    d = to_f64(boxes)
    want = Y.detect_decode(d, ax.double().numpy(), ay.double().numpy(), st.double().numpy())
    got = to_f64(out)
    s = st.double().numpy()
    mag_x = (np.abs(ax.double().numpy()) + d[:, 0] + d[:, 2]) * s
    mag_y = (np.abs(ay.double().numpy()) + d[:, 1] + d[:, 3]) * s
    tol = np.stack([mag_x, mag_y, mag_x, mag_y], axis=1) * 3 * U + 1e-30
    if dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(want)
    err = np.abs(got - want)
    assert np.all(np.isfinite(got))
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside the bound; worst "
                           f"{float((err / tol).max()):.3f}x")
    return got, want


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,A", [(64, 8400), (1, 8400), (3, 126), (2, 8404), (1, 1), (5, 7)])
def test_detect_decode_parity(B, A, dtype):
    _decode_case(B, A, dtype, seed=100 + A + B)


def test_detect_decode_small_image_grid():
    """A 96x64 image: 96 + 24 + 6 = 126 anchors over three strides (A % 4 != 0)."""
    grid = yi.anchor_grid(64, 96)
    assert grid[0].numel() == 126
    _decode_case(4, 126, torch.float32, seed=7, grid=grid)


def test_detect_decode_max_batch():
    """The largest batch the launch accepts (grid y = 65535), both vector widths."""
    for dtype in (torch.float32, torch.bfloat16):
        _decode_case(65535, 8, dtype, seed=11)


def test_detect_decode_exact_on_integers():
    """Integer distances and half-integer anchors at power-of-two strides are exact in
    float32: the result must equal the oracle bit for bit."""
    dev = device()
    A = 8400
    ax, ay, st = yi.anchor_grid()
    rng = np.random.default_rng(5)
    boxes = torch.from_numpy(rng.integers(0, 16, size=(8, 4, A)).astype(np.float32))
    announce("detect_decode integer distances")
    out = psa.detect_decode(boxes.to(dev), ax.to(dev), ay.to(dev), st.to(dev)).cpu()
    want = Y.detect_decode(boxes.double().numpy(), ax.double().numpy(), ay.double().numpy(),
                           st.double().numpy())
    assert np.array_equal(out.double().numpy(), want)


def _ciou_tols(p, g):
    M = np.max(np.abs(np.concatenate([p[:2] - p[2:] / 2, p[:2] + p[2:] / 2,
                                      g[:2] - g[2:] / 2, g[:2] + g[2:] / 2])), axis=0)
    smin = np.minimum(np.minimum(p[2], p[3]), np.minimum(g[2], g[3]))
    return M, smin


def _near_ties(p, g, margin=1e-3):
    px1, px2, py1, py2 = p[0] - p[2] / 2, p[0] + p[2] / 2, p[1] - p[3] / 2, p[1] + p[3] / 2
    gx1, gx2, gy1, gy2 = g[0] - g[2] / 2, g[0] + g[2] / 2, g[1] - g[3] / 2, g[1] + g[3] / 2
    gaps = [px1 - gx1, px2 - gx2, py1 - gy1, py2 - gy2,
            np.minimum(px2, gx2) - np.maximum(px1, gx1), np.minimum(py2, gy2) - np.maximum(py1, gy1)]
    return np.any(np.abs(np.stack(gaps)) < margin, axis=0)


def _ciou_case(pred, target, dloss, what, exact_ties=False):
    dev = device()
    N = pred.shape[1]
    announce(f"ciou {what} N={N}")
    pd, td, dd = pred.to(dev), target.to(dev), dloss.to(dev)
    loss, iou, v, alpha = psa.ciou_loss_fwd(pd, td)
    dpred = psa.ciou_loss_bwd(pd, td, iou, v, alpha, dd)
    torch.cuda.synchronize()
    p, g, dl = to_f64(pred), to_f64(target), to_f64(dloss)
    w_loss, w_iou, w_v, w_alpha = Y.ciou_forward(p, g)
    M, smin = _ciou_tols(p, g)
    tol = 32 * U * M / smin + 1e-6
    for name, got, want in (("loss", loss, w_loss), ("iou", iou, w_iou), ("v", v, w_v),
                            ("alpha", alpha, w_alpha)):
        got = to_f64(got)
        assert np.all(np.isfinite(got)), f"{what}: {name} not finite"
        err = np.abs(got - want)
        assert np.all(err <= tol), (f"{what}: {name} {np.sum(err > tol)} outside; worst "
                                    f"{float((err / tol).max()):.3f}x of the bound")
    # The backward is checked against the oracle's derivative at the oracle's own alpha.
    want_g = Y.ciou_backward(p, g, w_alpha, dl)
    got_g = to_f64(dpred)
    assert np.all(np.isfinite(got_g)), f"{what}: gradient not finite"
    # exact_ties: every edge pair is either equal in both precisions or far apart, so all
    # anchors are compared; otherwise anchors with an edge pair closer than 1e-3 are left out.
    ties = np.zeros(N, dtype=bool) if exact_ties else _near_ties(p, g)
    assert ties.mean() <= 1e-3, f"{what}: {ties.sum()} near-tie anchors"
    gtol = np.abs(dl) * (64 * U * M / smin ** 2 + 1e-5 * np.abs(want_g).max(axis=0)) + 1e-12
    err = np.abs(got_g - want_g)[:, ~ties]
    bad = err > gtol[~ties]
    assert not bad.any(), (f"{what}: gradient {bad.sum()} outside; worst "
                           f"{float((err / gtol[~ties]).max()):.3f}x of the bound")


@pytest.mark.parametrize("N", [64 * 8400, 8400, 4096 + 3, 5, 1, 4])
def test_ciou_parity(N):
    pred, target, dloss = yi.ciou_boxes(N, seed=200 + N % 97)
    _ciou_case(pred, target, dloss, f"random N={N}")


def test_ciou_identical_boxes():
    """Identical boxes: IoU 1, v 0, loss 0; every edge test is a tie that both sides take
    the same way, so the subgradient is compared in full."""
    _, target, dloss = yi.ciou_boxes(4096, seed=3)
    _ciou_case(target.clone(), target, dloss, "identical", exact_ties=True)
    # loss and IoU are within the float32 bound above (the corners round, so IoU may exceed 1
    # by a few ulp of M / s_min); the aspect term is exactly zero.
    loss, iou, v, alpha = psa.ciou_loss_fwd(target.to(device()), target.to(device()))
    assert float(v.abs().max()) == 0.0 and float(alpha.abs().max()) == 0.0


def test_ciou_disjoint_and_touching():
    """Disjoint pairs (no overlap) and pairs whose edges touch exactly (integer
    coordinates, so both precisions see the same tie)."""
    rng = np.random.default_rng(4)
    N = 2048
    tgt = np.stack([rng.integers(50, 500, N), rng.integers(50, 500, N),
                    2 * rng.integers(4, 40, N), 2 * rng.integers(4, 40, N)]).astype(np.float32)
    disjoint = tgt.copy()
    disjoint[0] += tgt[2] + 300
    _ciou_case(torch.from_numpy(disjoint), torch.from_numpy(tgt),
               torch.ones(N), "disjoint", exact_ties=True)
    touch = tgt.copy()
    touch[0] += tgt[2]          # shifted by its own width: the right edge of one is the left of the other
    pred = torch.from_numpy(touch)
    loss, iou, _, _ = psa.ciou_loss_fwd(pred.to(device()), torch.from_numpy(tgt).to(device()))
    assert float(iou.abs().max()) == 0.0
    _ciou_case(pred, torch.from_numpy(tgt), torch.ones(N), "touching", exact_ties=True)


def test_ciou_random_far_pairs():
    """Mostly non-overlapping pairs (IoU 0): the loss is driven by rho^2/c^2 and alpha v."""
    pred, target, dloss = yi.ciou_boxes(100_000, far=0.9, seed=9)
    _ciou_case(pred, target, dloss, "far")
