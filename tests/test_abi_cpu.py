"""The C ABI on the CPU: the library loads, exports what include/psa.h declares,
and rejects bad arguments before touching the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

import vision_transformer_attention_psapackqkv_amd as psa
from vision_transformer_attention_psapackqkv_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_binding.LIB_PATH), reason="libpsa.so not built")

A = 0x10000   # fake, 16-byte-aligned addresses: never dereferenced on these error paths
B_ = 0x90000000
C_ = 0xA0000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_0-9]+)\s*\(", text, flags=re.M))


def test_every_declared_symbol_is_exported_and_bound():
    lib = psa.load_library()
    names = declared_functions()
    assert names == set(_binding.SIGNATURES), names ^ set(_binding.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.psa_abi_version() == 4


def _status(fn, *args):
    lib = psa.load_library()
    st = getattr(lib, fn)(*args)
    return st, lib.psa_last_error().decode()


@pytest.mark.parametrize("fn", ["psa_pack_qkv", "psa_extract_v", "psa_merge_attn"])
def test_layout_argument_errors(fn):
    ok = dict(B=2, heads=2, kd=32, H=4, W=4, dt=1)

    def call(src=A, dst=B_, B=2, heads=2, kd=32, H=4, W=4, dt=1):
        return _status(fn, src, dst, B, heads, kd, H, W, dt, None)

    assert call(src=None) == (1, f"{fn}: input pointer is NULL")
    st, msg = call(dst=None)
    assert st == 1 and msg.startswith(fn)
    for bad in (dict(B=0), dict(heads=-1), dict(H=0), dict(W=-3)):
        st, msg = call(**bad)
        assert st == 2 and msg.startswith(fn + ":"), (bad, st, msg)
    for kd in (24, 8, 256, 1):
        st, msg = call(kd=kd)
        assert st == 3 and f"key_dim={kd}" in msg
    st, msg = call(dt=7)
    assert st == 3 and "dtype=7" in msg
    st, msg = call(src=A + 2)
    assert st == 4 and "aligned" in msg
    st, msg = call(dst=B_ + 8)
    assert st == 4
    st, msg = call(dst=A + 64)   # overlaps the input range
    assert st == 5 and "overlap" in msg
    assert ok  # silence linters


def test_fa2_fwd_argument_errors():
    def call(q=A, k=B_, v=C_, o=0xB0000000, lse=None, BH=2, nq=10, nk=12, D=64, s=0.125, dt=1,
             ws=None, wsb=0):
        return _status("fa2_fwd", q, k, v, o, lse, BH, nq, nk, D, ctypes.c_float(s), dt, ws, wsb, None)

    assert call(q=None)[0] == 1
    assert call(o=None)[0] == 1
    assert call(nq=0)[0] == 2
    assert call(BH=-1)[0] == 2
    st, msg = call(D=48)
    assert st == 3 and "head_dim=48" in msg and msg.startswith("fa2_fwd")
    assert call(s=0.0)[0] == 3
    assert call(s=float("nan"))[0] == 3
    assert call(s=-1.0)[0] == 3
    assert call(dt=2)[0] == 3
    assert call(v=C_ + 4)[0] == 4
    assert call(lse=0xC0000004)[0] == 4
    assert call(o=A)[0] == 5           # output aliases q
    assert call(lse=B_ + 16)[0] == 5   # lse inside k
    st, msg = call(ws=0xD0000008, wsb=4096)
    assert st == 4 and "workspace" in msg
    st, msg = call(ws=C_ + 64, wsb=4096)   # workspace inside v
    assert st == 5 and "workspace" in msg
    st, msg = call(ws=0xB0000000 - 1024, wsb=4096)   # workspace runs into o
    assert st == 5 and "workspace" in msg


def test_fa2_bwd_argument_errors():
    lib = psa.load_library()
    assert lib.fa2_bwd_workspace_bytes(256, 1600) == 2 * 256 * 1600 * 4
    assert lib.fa2_bwd_workspace_bytes(0, 5) == 0
    base = [0x1000000 * (i + 1) for i in range(10)]

    def call(ptrs=base, BH=2, nq=8, nk=8, D=32, s=0.2, dt=1):
        return _status("fa2_bwd", *ptrs, BH, nq, nk, D, ctypes.c_float(s), dt, None)

    for i in range(10):
        p = list(base)
        p[i] = None
        assert call(p)[0] == 1
    assert call(D=20)[0] == 3
    assert call(nk=0)[0] == 2
    p = list(base)
    p[6] = p[0]   # dq == q
    assert call(p)[0] == 5
    p = list(base)
    p[9] = p[7]   # workspace == dk
    assert call(p)[0] == 5


def test_fused_argument_errors():
    def call(x=A, out=B_, v=None, lse=None, B=1, h=2, kd=64, H=5, W=5, s=0.125, dt=1, ws=None, wsb=0):
        return _status("psa_attention_fwd", x, out, v, lse, B, h, kd, H, W, ctypes.c_float(s), dt,
                       ws, wsb, None)

    assert call(x=None)[0] == 1
    assert call(out=None)[0] == 1
    assert call(H=0)[0] == 2
    assert call(kd=96)[0] == 3
    assert call(s=float("inf"))[0] == 3
    assert call(v=C_ + 2)[0] == 4
    assert call(v=B_)[0] == 5           # V residual aliases out
    st, msg = call(out=A + 16)
    assert st == 5 and msg.startswith("psa_attention_fwd")
    assert call(ws=C_ + 4, wsb=64)[0] == 4
    st, msg = call(ws=B_ + 32, wsb=64)   # workspace inside out
    assert st == 5 and "workspace" in msg


def test_forward_workspace_bytes_without_a_device():
    """Invalid sizes and float32 ask for no workspace; without a GPU no launch is
    sized, so no split is planned either."""
    lib = psa.load_library()
    assert lib.fa2_fwd_workspace_bytes(0, 10, 10, 64, 1) == 0
    assert lib.fa2_fwd_workspace_bytes(2, 10, 10, 48, 1) == 0
    assert lib.fa2_fwd_workspace_bytes(32, 6400, 6400, 64, 0) == 0
    assert lib.fa2_fwd_workspace_bytes(2, 10, 10, 64, 9) == 0
    assert lib.psa_attention_fwd_workspace_bytes(4, 8, 24, 80, 80, 1) == 0
    assert lib.psa_attention_fwd_workspace_bytes(4, 8, 64, 80, 80, 0) == 0
    assert lib.psa_attention_fwd_workspace_bytes(-1, 8, 64, 80, 80, 1) == 0


def test_error_string_cleared_on_next_error_free_path():
    lib = psa.load_library()
    lib.psa_pack_qkv(None, B_, 1, 1, 16, 1, 1, 1, None)
    assert lib.psa_last_error().decode() != ""
    # workspace-size query does not touch the error state; a later error overwrites it
    lib.psa_merge_attn(A, None, 1, 1, 16, 1, 1, 1, None)
    assert lib.psa_last_error().decode().startswith("psa_merge_attn")


def test_psa_attention_bwd_argument_errors():
    lib = psa.load_library()
    assert lib.psa_attention_bwd_workspace_bytes(32, 8, 40, 40) == 2 * 256 * 1600 * 4
    assert lib.psa_attention_bwd_workspace_bytes(0, 8, 40, 40) == 0
    base = [0x1000000 * (i + 1) for i in range(7)]   # qkv, out, lse, dout, dv, dqkv, workspace

    def call(ptrs=base, B=1, h=2, kd=32, H=4, W=4, s=0.2, dt=1):
        return _status("psa_attention_bwd", *ptrs, B, h, kd, H, W, ctypes.c_float(s), dt, None)

    for i in (0, 1, 2, 3, 5, 6):
        p = list(base)
        p[i] = None
        st, msg = call(p)
        assert st == 1 and msg.startswith("psa_attention_bwd"), (i, st, msg)
    p = list(base)
    p[4] = None                       # no residual gradient: valid, so the failure is elsewhere
    assert call(p, kd=24)[0] == 3
    assert call(kd=48)[0] == 3
    st, msg = call(dt=7)
    assert st == 3 and "dtype=7" in msg
    assert call(H=0)[0] == 2
    assert call(s=float("nan"))[0] == 3
    p = list(base)
    p[3] = base[3] + 2
    assert call(p)[0] == 4
    p = list(base)
    p[5] = base[0]                    # dqkv aliases qkv
    assert call(p)[0] == 5
    p = list(base)
    p[6] = base[5] + 64               # workspace inside dqkv
    assert call(p)[0] == 5


def test_detect_decode_argument_errors():
    base = [0x1000000 * (i + 1) for i in range(5)]   # boxes, anchor_x, anchor_y, strides, out

    def call(ptrs=base, B=2, A=100, dt=0):
        return _status("detect_decode", *ptrs, B, A, dt, None)

    for i in range(5):
        p = list(base)
        p[i] = None
        st, msg = call(p)
        assert st == 1 and msg.startswith("detect_decode"), (i, st, msg)
    assert call(B=0)[0] == 2
    assert call(A=0)[0] == 2
    assert call(B=70000)[0] == 2
    st, msg = call(dt=5)
    assert st == 3 and "dtype=5" in msg
    for i in range(5):
        p = list(base)
        p[i] += 4
        assert call(p)[0] == 4, i
    p = list(base)
    p[4] = base[0] + 16                   # out inside boxes (2*4*100 floats)
    st, msg = call(p)
    assert st == 5 and "out" in msg
    p = list(base)
    p[4] = base[3] - 3200 + 16            # out runs into strides
    assert call(p)[0] == 5


def test_ciou_argument_errors():
    fwd = [0x1000000 * (i + 1) for i in range(6)]   # pred, target, loss, iou, v, alpha
    bwd = [0x1000000 * (i + 1) for i in range(7)]   # pred, target, iou, v, alpha, dloss, dpred

    def call_f(ptrs=fwd, N=64):
        return _status("ciou_loss_fwd", *ptrs, N, None)

    def call_b(ptrs=bwd, N=64):
        return _status("ciou_loss_bwd", *ptrs, N, None)

    for call, base, fn in ((call_f, fwd, "ciou_loss_fwd"), (call_b, bwd, "ciou_loss_bwd")):
        for i in range(len(base)):
            p = list(base)
            p[i] = None
            st, msg = call(p)
            assert st == 1 and msg.startswith(fn), (fn, i, st, msg)
            p = list(base)
            p[i] += 8
            assert call(p)[0] == 4, (fn, i)
        assert call(N=0)[0] == 2
        assert call(N=-5)[0] == 2
        assert call(N=1 << 40)[0] == 2
    p = list(fwd)
    p[3] = p[2] + 16                      # iou overlaps loss
    st, msg = call_f(p)
    assert st == 5 and "iou" in msg and "loss" in msg
    p = list(fwd)
    p[5] = p[0] + 512                     # alpha inside pred (4*64 floats)
    assert call_f(p)[0] == 5
    p = list(bwd)
    p[6] = p[5]                           # dpred aliases dloss
    assert call_b(p)[0] == 5


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipGetErrorString.restype = ctypes.c_char_p
    return lib


def test_rejected_call_leaves_a_stale_hip_error_alone():
    """A HIP error left by an earlier, unrelated call on this thread: an entry point that rejects
    its arguments launches nothing, reports its own validation failure and leaves that error for
    the caller to read. (That a launching entry point clears such an error first, so it is not
    reported as the entry point's launch failure, needs a GPU: tests/test_layout_gpu.py.)"""
    hip = _hip()
    stale = hip.hipSetDevice(9999)
    assert stale != 0
    st, msg = _status("psa_pack_qkv", A, B_, 2, 2, 24, 4, 4, 1, None)
    assert st == 3 and msg == "psa_pack_qkv: key_dim=24 is not one of 16, 32, 64, 128"
    assert hip.hipGetLastError() == stale


def test_fa2_bwd_noalloc_argument_errors():
    """The allocation-free FA2 backward: same argument checks as fa2_bwd, no workspace, and a
    call larger than the library's scratch is rejected before anything is launched."""
    p = [A + i * 0x100000 for i in range(9)]

    def call(ptrs=p, BH=4, n_q=64, n_k=64, D=32, scale=0.125, dt=1):
        return _status("fa2_bwd_noalloc", *ptrs, BH, n_q, n_k, D, scale, dt, None)

    st, msg = call(ptrs=p[:8] + [None])
    assert st == 1 and msg == "fa2_bwd_noalloc: every pointer argument is required"
    st, msg = call(D=48)
    assert st == 3 and "head_dim=48" in msg
    st, msg = call(BH=0)
    assert st == 2 and msg.startswith("fa2_bwd_noalloc:")
    limit = (16 << 20) // 8
    st, msg = call(BH=2, n_q=limit // 2 + 1, n_k=8)
    assert st == 2 and "scratch" in msg and str(16 << 20) in msg, msg
    st, msg = call(ptrs=p[:6] + [p[0]] + p[7:])
    assert st == 5 and "overlap" in msg


def test_attention_rows_beyond_one_launch_are_rejected():
    """The attention kernels give every 128 rows one workgroup and a launch holds fewer than
    2^32 work-items, so BH * n (rounded up to 128) must stay below 2^31 - 2^23; larger calls
    fail with PSA_ERR_SHAPE before anything is launched, naming the entry point."""
    big_bh, big_n = 1 << 14, 1 << 17            # 2^31 rows
    st, msg = _status("fa2_fwd", A, B_, C_, 0xB0000000, None, big_bh, big_n, 64, 16,
                      ctypes.c_float(0.25), 1, None, 0, None)
    assert st == 2 and msg.startswith("fa2_fwd") and "one launch" in msg, msg
    st, msg = _status("fa2_fwd", A, B_, C_, 0xB0000000, None, big_bh, 64, big_n, 16,
                      ctypes.c_float(0.25), 1, None, 0, None)   # many keys: the dK/dV grid's rows
    assert st == 2 and "one launch" in msg, msg
    base = [0x1000000 * (i + 1) for i in range(10)]
    st, msg = _status("fa2_bwd", *base, big_bh, big_n, big_n, 16, ctypes.c_float(0.25), 1, None)
    assert st == 2 and msg.startswith("fa2_bwd") and "one launch" in msg, msg
    # B * heads = 8192 maps of 512 x 512 pixels: 2^31 rows
    st, msg = _status("psa_attention_fwd", A, B_, None, None, 1024, 8, 16, 512, 512,
                      ctypes.c_float(0.25), 1, None, 0, None)
    assert st == 2 and msg.startswith("psa_attention_fwd") and "one launch" in msg, msg
    bp = [0x1000000 * (i + 1) for i in range(7)]
    st, msg = _status("psa_attention_bwd", *bp, 1024, 8, 16, 512, 512, ctypes.c_float(0.25), 1, None)
    assert st == 2 and msg.startswith("psa_attention_bwd") and "one launch" in msg, msg
    # just under the limit passes the size checks (and fails later, on the aliasing of the
    # fake pointers, which shows the size check let it through)
    ok_n = ((1 << 31) - (1 << 23)) // (1 << 14) - 128   # a multiple of 128 below the limit
    st, msg = _status("fa2_fwd", A, A, A, A, None, 1 << 14, ok_n, 64, 16, ctypes.c_float(0.25), 1,
                      None, 0, None)
    assert st == 5, msg
