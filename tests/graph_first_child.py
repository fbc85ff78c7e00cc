"""Child process of test_graph_gpu.py: the library's first calls in a process made under HIP
graph capture.

Every entry point runs a per-device set-up on its first call on a device (it looks up the
device address of fa2_bwd_noalloc's scratch array). Here that first call is inside
torch.cuda.graph capture: the captured fused forward, FA2 forward and fa2_bwd_noalloc are
replayed three times, and every replay must equal the same calls made eagerly afterwards,
bit for bit. Prints "ALL OK" at the end; exits non-zero on a mismatch.
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import torch  # noqa: E402

import psa_inputs as I  # noqa: E402
import vision_transformer_attention_psapackqkv_amd as psa  # noqa: E402


def main():
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, h, KD, H, W = 2, 2, 32, 16, 16
    x = I.make_qkv(B, h, KD, H, W, seed=61).to(dev)
    q, k, v, do = (t.to(dev) for t in I.make_attention_inputs(4, 300, 300, 32, seed=62, with_dout=True))
    out = torch.empty((B, 2 * h * KD, H, W), dtype=x.dtype, device=dev)
    vres, lse = torch.empty_like(out), torch.empty((B * h, H * W), dtype=torch.float32, device=dev)
    o, l2 = torch.empty_like(q), torch.empty((4, 300), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()

    def calls():
        psa.psa_attention_fwd(x, h, KD, out=out, v_out=vres, lse=lse)
        psa.fa2_fwd(q, k, v, out=o, lse=l2)
        psa.fa2_bwd_noalloc(q, k, v, o, do, l2, dq=dq, dk=dk, dv=dv)

    print("[graph-first] capturing the first library calls of the process", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    outs = (out, vres, lse, o, l2, dq, dk, dv)
    replays = []
    for _ in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replays.append([t.clone() for t in outs])
    calls()
    torch.cuda.synchronize()
    for i, rep in enumerate(replays):
        for got, want in zip(rep, outs):
            if not torch.equal(got, want):
                print(f"[graph-first] replay {i} differs from the eager calls", flush=True)
                return 1
    print("ALL OK", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
