"""The forward and the PSA backward captured in a HIP graph (torch.cuda.CUDAGraph over the
library's C calls on the capturing stream): every replay equals the eager launch. The
launches allocate nothing and enqueue no memset, so they can be captured as they are."""
import pytest
import torch

import psa_inputs as I
import vision_transformer_attention_psapackqkv_amd as psa
from tests.gpu_helpers import announce, device

pytestmark = pytest.mark.gpu


def _replays_match(graph, outputs, eager, churn):
    for i in range(3):
        for t in outputs:
            t.zero_()
        churn()                       # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, eager):
            assert torch.equal(got, want), f"replay {i} differs from the eager launch"


def test_psa_attention_fwd_in_a_graph():
    dev = device()
    B, h, KD, H, W = 4, 8, 64, 80, 80     # the benchmark map: its grid splits the last round
    announce("psa_attention_fwd graph capture")
    x = I.make_qkv(B, h, KD, H, W, seed=41).to(dev)
    ws = torch.empty(psa.psa_attention_fwd_workspace_bytes(B, h, KD, H, W), dtype=torch.uint8, device=dev)
    out = torch.empty((B, 2 * h * KD, H, W), dtype=x.dtype, device=dev)
    vres, lse = torch.empty_like(out), torch.empty((B * h, H * W), dtype=torch.float32, device=dev)
    e_out, e_v, e_lse = psa.psa_attention_fwd(x, h, KD, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):        # warm-up on the side stream before capture
        psa.psa_attention_fwd(x, h, KD, out=out, v_out=vres, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        psa.psa_attention_fwd(x, h, KD, out=out, v_out=vres, lse=lse, workspace=ws)
    y = torch.randn(1 << 20, device=dev)

    def churn():
        psa.psa_pack_qkv(x, h, KD)
        y.mul_(1.5)
    _replays_match(g, [out, vres, lse], [e_out, e_v, e_lse], churn)


def test_psa_attention_bwd_in_a_graph():
    dev = device()
    B, h, KD, H, W = 2, 4, 32, 24, 24
    announce("psa_attention_bwd graph capture")
    x = I.make_qkv(B, h, KD, H, W, seed=42).to(dev)
    out, _, lse = psa.psa_attention_fwd(x, h, KD, want_v=False)
    g_out = torch.randn(out.shape, device=dev).to(out.dtype)
    g_v = torch.randn(out.shape, device=dev).to(out.dtype)
    ws = torch.empty((psa.load_library().psa_attention_bwd_workspace_bytes(B, h, H, W) // 4,),
                     dtype=torch.float32, device=dev)
    dqkv = torch.empty_like(x)
    eager = psa.psa_attention_bwd(x, out, lse, g_out, h, KD, dv=g_v, workspace=ws).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        psa.psa_attention_bwd(x, out, lse, g_out, h, KD, dv=g_v, dqkv=dqkv, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        psa.psa_attention_bwd(x, out, lse, g_out, h, KD, dv=g_v, dqkv=dqkv, workspace=ws)
    _replays_match(g, [dqkv], [eager], lambda: psa.psa_attention_fwd(x, h, KD, want_v=False))


def test_detect_decode_and_ciou_in_a_graph():
    """Detect-decode (both dtypes) and the CIoU forward and backward in one captured graph."""
    import yolo_inputs as yi
    dev = device()
    announce("detect_decode + ciou graph capture")
    ax, ay, st = (t.to(dev) for t in yi.anchor_grid())
    boxes = {dt: yi.ltrb_boxes(8, 8400, dtype=dt, seed=43).to(dev) for dt in (torch.float32, torch.bfloat16)}
    dec = {dt: torch.empty_like(b) for dt, b in boxes.items()}
    N = 8 * 8400 + 3                  # ragged: the one-anchor-per-lane kernels
    p, t, dl = (x.to(dev) for x in yi.ciou_boxes(N, seed=44))
    fwd = tuple(torch.empty(N, device=dev) for _ in range(4))
    dp = torch.empty((4, N), device=dev)
    eager = [psa.detect_decode(b, ax, ay, st) for b in boxes.values()]
    e_fwd = psa.ciou_loss_fwd(p, t)
    eager += list(e_fwd) + [psa.ciou_loss_bwd(p, t, e_fwd[1], e_fwd[2], e_fwd[3], dl)]

    def launches():
        for dt, b in boxes.items():
            psa.detect_decode(b, ax, ay, st, out=dec[dt])
        psa.ciou_loss_fwd(p, t, out=fwd)
        psa.ciou_loss_bwd(p, t, fwd[1], fwd[2], fwd[3], dl, dpred=dp)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launches()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launches()
    y = torch.randn(1 << 20, device=dev)
    _replays_match(g, list(dec.values()) + list(fwd) + [dp], eager, lambda: y.mul_(1.5))


def test_fa2_and_layout_in_a_graph():
    """The unfused chain's calls (pack, fa2_fwd on both V halves with the tail-split
    workspace, merge, extract) and the FA2 backward through fa2_bwd_noalloc, the entry point
    meant for capture (it allocates nothing: its -Delta rows live in the library's scratch),
    in one captured graph."""
    dev = device()
    B, h, KD, H, W = 2, 8, 64, 80, 80     # the FA2 grid splits its last round
    announce("pack + fa2_fwd x2 + merge + extract + fa2_bwd_noalloc graph capture")
    x = I.make_qkv(B, h, KD, H, W, seed=45).to(dev)
    BH, N = B * h, H * W
    packed = torch.empty((4, BH, N, KD), dtype=x.dtype, device=dev)
    o2 = torch.empty((2, BH, N, KD), dtype=x.dtype, device=dev)
    lse = torch.empty((BH, N), dtype=torch.float32, device=dev)
    merged = torch.empty((B, 2 * h * KD, H, W), dtype=x.dtype, device=dev)
    vres = torch.empty_like(merged)
    ws = torch.empty(psa.fa2_fwd_workspace_bytes(BH, N, N, KD), dtype=torch.uint8, device=dev)
    assert ws.numel() > 0
    dout = torch.randn((BH, N, KD), device=dev).to(x.dtype)
    grads = [torch.empty((BH, N, KD), dtype=x.dtype, device=dev) for _ in range(3)]

    def launches():
        psa.psa_pack_qkv(x, h, KD, out=packed)
        psa.fa2_fwd(packed[0], packed[1], packed[2], out=o2[0], lse=lse, workspace=ws)
        psa.fa2_fwd(packed[0], packed[1], packed[3], out=o2[1], want_lse=False, workspace=ws)
        psa.psa_merge_attn(o2, B, h, KD, H, W, out=merged)
        psa.psa_extract_v(packed, B, h, KD, H, W, out=vres)
        psa.fa2_bwd_noalloc(packed[0], packed[1], packed[2], o2[0], dout, lse,
                            dq=grads[0], dk=grads[1], dv=grads[2])
    launches()
    torch.cuda.synchronize()
    eager = [t.clone() for t in [packed, o2, lse, merged, vres] + grads]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launches()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launches()
    y = torch.randn(1 << 20, device=dev)
    _replays_match(g, [packed, o2, lse, merged, vres] + grads, eager, lambda: y.mul_(1.5))


def test_first_library_calls_under_capture():
    """In a fresh process, the library's first calls (which run its per-device set-up) are made
    under graph capture; the replays equal the eager calls (`graph_first_child.py`)."""
    import os
    import subprocess
    import sys
    device()
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "graph_first_child.py")
    announce("first library calls of a process under graph capture (child process)")
    r = subprocess.run([sys.executable, "-u", child], capture_output=True, text=True, timeout=240)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, f"child exited {r.returncode}"
    assert "ALL OK" in r.stdout
