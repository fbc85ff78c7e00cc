"""FA2 forward and the fused PSA forward on the GPU against the float64 oracle."""
import numpy as np
import pytest
import torch

import psa_inputs as I
import vision_transformer_attention_psapackqkv_amd as psa
from oracle import psa_oracle as O
from tests.gpu_helpers import (announce, assert_attention_close, assert_lse_close, bits, device,
                               to_f64)

pytestmark = pytest.mark.gpu

# (BH, n_q, n_k, head_dim, dtype): several query/key tiles with ragged tails.
FA2_SHAPES = [
    (1, 1, 1, 32, "bf16"),
    (2, 64, 64, 16, "bf16"),
    (3, 100, 77, 32, "bf16"),
    (2, 129, 200, 64, "bf16"),
    (2, 65, 63, 128, "bf16"),
    (32, 400, 400, 32, "bf16"),
    (1, 300, 1, 64, "bf16"),
    (2, 64, 64, 16, "f32"),
    (3, 100, 77, 32, "f32"),
    (2, 33, 130, 64, "f32"),
    (1, 20, 45, 128, "f32"),
    # float32 with fewer keys than a row's four lanes (lanes that never see a key), and
    # key counts that end a 32-key tile after 1..3 of a lane's keys
    (2, 37, 1, 16, "f32"),
    (1, 5, 2, 32, "f32"),
    (2, 70, 3, 64, "f32"),
    (1, 33, 5, 128, "f32"),
    (3, 45, 34, 16, "f32"),
    (2, 31, 67, 64, "f32"),
]


def _fa2_id(s):
    return "BH{}_q{}_k{}_d{}_{}".format(*s)


@pytest.mark.parametrize("shape", FA2_SHAPES, ids=_fa2_id)
def test_fa2_fwd(shape):
    dev = device()
    BH, nq, nk, D, dt = shape
    announce(f"fa2_fwd {_fa2_id(shape)}")
    q, k, v = I.make_attention_inputs(BH, nq, nk, D, dtype=dt, seed=BH + nq + nk + D)
    s = D ** -0.5
    o, lse = psa.fa2_fwd(q.to(dev), k.to(dev), v.to(dev), scale=s)
    want_o, want_lse = O.attention(to_f64(q), to_f64(k), to_f64(v), s)
    assert_attention_close(to_f64(o), want_o, dt, "fa2_fwd O")
    assert_lse_close(to_f64(lse), want_lse, dt, "fa2_fwd")


# (B, heads, key_dim, H, W, dtype)
PSA_SHAPES = [
    (1, 1, 16, 8, 8, "f32"),            # the tiny float32 map
    (8, 4, 32, 20, 20, "bf16"),         # the 20x20 map, whole
    (1, 2, 16, 1, 1, "bf16"),           # one pixel: O = V
    (2, 1, 32, 7, 9, "bf16"),           # N = 63, not a multiple of 8
    (1, 2, 64, 5, 13, "bf16"),          # N = 65
    (1, 1, 128, 9, 12, "bf16"),         # key_dim 128, N = 108
    (2, 2, 64, 16, 16, "bf16"),         # N = 256, whole tiles
    (1, 2, 32, 3, 3, "f32"),
    (1, 1, 64, 10, 13, "f32"),
    (1, 1, 128, 4, 6, "f32"),
    (1, 2, 16, 1, 1, "f32"),            # one pixel in float32: O = V
    (2, 1, 32, 1, 3, "f32"),            # N = 3: a row's fourth lane sees no key
    (1, 1, 64, 5, 7, "f32"),            # N = 35: a second tile of 3 keys
]


def _psa_id(s):
    return "B{}h{}kd{}_{}x{}_{}".format(*s)


def _check_psa(qkv, B, h, KD, H, W, dt, out, vres, lse, bh_sel=None):
    x = to_f64(qkv)
    if bh_sel is None:
        want_out, want_v, want_lse = O.psa_forward(x, B, h, KD, H, W)
        got_out = to_f64(out)
        got_lse = to_f64(lse)
    else:
        # sampled batch-heads: the oracle's attention on those heads' packed slices
        packed = O.pack_qkv(x, B, h, KD, H, W)
        s = O.default_scale(KD)
        o_lo, want_lse = O.attention(packed[0][bh_sel], packed[1][bh_sel], packed[2][bh_sel], s)
        o_hi, _ = O.attention(packed[0][bh_sel], packed[1][bh_sel], packed[3][bh_sel], s)
        want_out = np.concatenate([o_lo, o_hi], axis=2)             # [S, N, 2KD]
        got = to_f64(out).reshape(B * h, 2 * KD, H * W)[bh_sel]      # [S, 2KD, N]
        got_out = got.transpose(0, 2, 1)
        got_lse = to_f64(lse)[bh_sel]
        want_v = None
    assert_attention_close(got_out, want_out, dt, "psa_attention_fwd out")
    assert_lse_close(got_lse, want_lse, dt, "psa_attention_fwd")
    # the V residual is a bit copy of the V channels
    want_v_bits = O.extract_v(O.pack_qkv(bits(qkv), B, h, KD, H, W), B, h, KD, H, W)
    assert np.array_equal(bits(vres), want_v_bits), "V residual differs"
    return want_v


@pytest.mark.parametrize("shape", PSA_SHAPES, ids=_psa_id)
def test_psa_fused_fwd(shape):
    dev = device()
    B, h, KD, H, W, dt = shape
    announce(f"psa_attention_fwd {_psa_id(shape)}")
    qkv = I.make_qkv(B, h, KD, H, W, dtype=dt, dist="uniform" if dt == "f32" else "normal",
                     seed=11 * B + h + KD + H * W)
    out, vres, lse = psa.psa_attention_fwd(qkv.to(dev), h, KD)
    _check_psa(qkv, B, h, KD, H, W, dt, out, vres, lse)


@pytest.mark.parametrize("shape", PSA_SHAPES, ids=_psa_id)
def test_psa_unfused_fwd(shape):
    """pack -> fa2_fwd(V_lo) -> fa2_fwd(V_hi) -> merge, plus extract, as separate launches."""
    dev = device()
    B, h, KD, H, W, dt = shape
    announce(f"psa unfused {_psa_id(shape)}")
    qkv = I.make_qkv(B, h, KD, H, W, dtype=dt, dist="uniform" if dt == "f32" else "normal",
                     seed=11 * B + h + KD + H * W)
    packed = psa.psa_pack_qkv(qkv.to(dev), h, KD)
    o2 = torch.empty((2,) + tuple(packed.shape[1:]), dtype=packed.dtype, device=dev)
    _, lse = psa.fa2_fwd(packed[0], packed[1], packed[2], out=o2[0])
    psa.fa2_fwd(packed[0], packed[1], packed[3], out=o2[1], want_lse=False)
    out = psa.psa_merge_attn(o2, B, h, KD, H, W)
    vres = psa.psa_extract_v(packed, B, h, KD, H, W)
    _check_psa(qkv, B, h, KD, H, W, dt, out, vres, lse)


@pytest.mark.parametrize("name", ["psa_fwd_bf16_20x20", "psa_fwd_bf16_40x40_peaked", "psa_fwd_bf16_80x80"])
def test_psa_fused_workloads(name):
    """The workload maps at full size through the fused entry point in the launch the benchmark
    times (with its tail-split workspace), every query row of the checked batch-heads: all of them
    up to 32 (the 80x80 map: every head that holds split tail tiles), else 32 spread over the map
    (every 8th at 40x40, so each XCD's contiguous run of query tiles is checked several times)."""
    dev = device()
    w = I.WORKLOADS[name]
    announce(f"psa_attention_fwd workload {name}")
    qkv = I.make_workload_qkv(w)
    ws = torch.empty(psa.psa_attention_fwd_workspace_bytes(w.B, w.heads, w.key_dim, w.H, w.W),
                     dtype=torch.uint8, device=dev)
    out, vres, lse = psa.psa_attention_fwd(qkv.to(dev), w.heads, w.key_dim, workspace=ws)
    sel = np.arange(w.BH) if w.BH <= 32 else np.unique(np.append(np.arange(0, w.BH, w.BH // 32), w.BH - 1))
    _check_psa(qkv, w.B, w.heads, w.key_dim, w.H, w.W, w.dtype, out, vres, lse, bh_sel=sel)


def test_psa_fused_repeatable_and_matches_halves():
    """Two runs give identical bits; the first half equals an FA2 run on (Q, K, V_lo)
    to within bf16 tolerance (the fused softmax is shared by both halves)."""
    dev = device()
    B, h, KD, H, W = 2, 2, 32, 12, 12
    announce("psa fused repeatability")
    qkv = I.make_qkv(B, h, KD, H, W, seed=77).to(dev)
    o1, _, l1 = psa.psa_attention_fwd(qkv, h, KD)
    o2, _, l2 = psa.psa_attention_fwd(qkv, h, KD)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    packed = psa.psa_pack_qkv(qkv, h, KD)
    lo, lse_lo = psa.fa2_fwd(packed[0], packed[1], packed[2])
    lo_nchw = to_f64(o1).reshape(B * h, 2 * KD, H * W)[:, :KD].transpose(0, 2, 1)
    assert_attention_close(lo_nchw, to_f64(lo), "bf16", "fused lo half vs fa2_fwd")
    assert np.abs(to_f64(lse_lo) - to_f64(l1)).max() < 5e-3


# Grids that leave a short partial last round of workgroups on a 256-CU gfx950
# (80x80 maps at batch 2 and 4, key_dim 128 at batch 4, a 48x48 map with
# key_dim 32 at batch 8): given a workspace, the launch cuts those last query
# tiles into key-range pieces and merges them in a second kernel. Checked on
# the first head and the last two (whose tiles are all in the last round),
# every query row, and against the same launch run unsplit. The 44x48 maps
# (N = 2112, 16.5 query tiles per batch-head) put a half-empty query tile, whose
# last two waves hold no query, among the split tiles of the last batch-head.
TAIL_PSA = [
    (2, 8, 64, 80, 80),
    (4, 4, 128, 80, 80),
    (8, 8, 32, 48, 48),
    (8, 8, 32, 44, 48),
    (12, 8, 64, 44, 48),
]


@pytest.mark.parametrize("shape", TAIL_PSA, ids=lambda s: "B{}h{}kd{}_{}x{}".format(*s))
def test_psa_fused_tail_split(shape):
    dev = device()
    B, h, KD, H, W = shape
    announce(f"psa_attention_fwd tail split B{B}h{h}kd{KD}_{H}x{W}")
    nbytes = psa.psa_attention_fwd_workspace_bytes(B, h, KD, H, W)
    assert nbytes > 0, "this grid is expected to split its last round on a 256-CU gfx950"
    qkv = I.make_qkv(B, h, KD, H, W, seed=5 * B + KD + H)
    x = qkv.to(dev)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out, vres, lse = psa.psa_attention_fwd(x, h, KD, workspace=ws)
    sel = np.array([0, B * h - 2, B * h - 1])
    _check_psa(qkv, B, h, KD, H, W, "bf16", out, vres, lse, bh_sel=sel)
    # a second call on the same workspace gives the same bits
    out2, _, lse2 = psa.psa_attention_fwd(x, h, KD, workspace=ws)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # unsplit (no workspace, or 16 bytes short): the same bits either way, and close
    # to the split run. The two differ only in how P is rounded to bf16 (each piece
    # rounds against its own running max), so O within one bf16 step and LSE within
    # 1e-3 (relative error of the row sum).
    empty = torch.empty(0, dtype=torch.uint8, device=dev)
    short = ws[: nbytes - 16]
    o_none, _, l_none = psa.psa_attention_fwd(x, h, KD, workspace=empty)
    o_short, _, l_short = psa.psa_attention_fwd(x, h, KD, workspace=short)
    assert torch.equal(o_none, o_short) and torch.equal(l_none, l_short)
    diff = (o_none.float() - out.float()).abs()
    assert diff.max().item() <= 2.0 ** -7 * max(1.0, out.float().abs().max().item())
    assert (l_none - lse).abs().max().item() < 1e-3


@pytest.mark.parametrize("shape", [(32, 6400, 64), (48, 2112, 64)], ids=lambda s: "BH{}n{}d{}".format(*s))
def test_fa2_fwd_tail_split(shape):
    """FA2 forward on packed [BH, n, D] tensors whose grid leaves a short last round,
    checked on the last two batch-heads (n = 2112: a half-empty last query tile among
    the split tiles)."""
    dev = device()
    BH, n, D = shape
    announce(f"fa2_fwd tail split BH{BH} n{n} d{D}")
    assert psa.fa2_fwd_workspace_bytes(BH, n, n, D) > 0
    q, k, v = I.make_attention_inputs(BH, n, n, D, seed=31)
    o, lse = psa.fa2_fwd(q.to(dev), k.to(dev), v.to(dev))
    sel = [BH - 2, BH - 1]
    want_o, want_lse = O.attention(to_f64(q)[sel], to_f64(k)[sel], to_f64(v)[sel], D ** -0.5)
    assert_attention_close(to_f64(o)[sel], want_o, "bf16", "fa2_fwd tail O")
    assert_lse_close(to_f64(lse)[sel], want_lse, "bf16", "fa2_fwd tail")


@pytest.mark.parametrize("shape", [(32, 6400, 4096, 64), (48, 2112, 3000, 64)],
                         ids=lambda s: "BH{}q{}k{}d{}".format(*s))
def test_fa2_fwd_tail_split_cross_lengths(shape):
    """The tail split with n_q != n_k: pieces cut the key range of n_k keys while the split
    tiles are counted over n_q queries; checked on the last two batch-heads and against the
    same launch run unsplit."""
    dev = device()
    BH, nq, nk, D = shape
    announce(f"fa2_fwd tail split BH{BH} q{nq} k{nk} d{D}")
    nbytes = psa.fa2_fwd_workspace_bytes(BH, nq, nk, D)
    assert nbytes > 0, "this grid is expected to split its last round on a 256-CU gfx950"
    q, k, v = I.make_attention_inputs(BH, nq, nk, D, seed=37)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    o, lse = psa.fa2_fwd(qd, kd, vd, workspace=ws)
    sel = [BH - 2, BH - 1]
    want_o, want_lse = O.attention(to_f64(q)[sel], to_f64(k)[sel], to_f64(v)[sel], D ** -0.5)
    assert_attention_close(to_f64(o)[sel], want_o, "bf16", "fa2_fwd tail O (n_q != n_k)")
    assert_lse_close(to_f64(lse)[sel], want_lse, "bf16", "fa2_fwd tail (n_q != n_k)")
    o_none, l_none = psa.fa2_fwd(qd, kd, vd, workspace=torch.empty(0, dtype=torch.uint8, device=dev))
    assert (o_none.float() - o.float()).abs().max().item() <= 2.0 ** -7 * max(1.0, o.float().abs().max().item())
    assert (l_none - lse).abs().max().item() < 1e-3


@pytest.mark.parametrize("hw", [(1448, 1448), (1449, 1449)], ids=lambda s: "{}x{}".format(*s))
def test_psa_fused_fwd_largest_slab(hw):
    """The fused forward at the edge of its 32-bit buffer offsets: a key_dim-128 map whose
    batch-head slab of Q, K, V_lo, V_hi is just under 2 GB (1448x1448: staged straight into
    LDS with buffer loads) and just over it (1449x1449, N not a multiple of 8 either: staged
    through registers with 64-bit addresses). 16 sampled pixels against the oracle (both
    halves and the LSE, all 2.1 M keys); the V residual bit-exact on the whole map."""
    dev = device()
    H, W = hw
    B, h, KD = 1, 1, 128
    N = H * W
    announce(f"psa_attention_fwd largest slab {H}x{W} key_dim {KD}")
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    qkv = torch.randn((B, 4 * h * KD, H, W), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    out, vres, lse = psa.psa_attention_fwd(qkv, h, KD)
    torch.cuda.synchronize()
    assert torch.equal(vres, qkv[:, 2 * KD:4 * KD]), "V residual differs"
    rows = np.linspace(0, N - 1, 16).astype(np.int64)
    x = qkv.reshape(4, KD, N)
    q = to_f64(x[0][:, torch.from_numpy(rows).to(dev)].t())[None]      # [1, 16, KD]
    k = to_f64(x[1].t())[None]                                          # [1, N, KD]
    want_lse = None
    for j in range(2):
        v = to_f64(x[2 + j].t())[None]
        want_o, want_lse = O.attention(q, k, v, KD ** -0.5)
        got = to_f64(out.reshape(2, KD, N)[j][:, torch.from_numpy(rows).to(dev)].t())[None]
        assert_attention_close(got, want_o, "bf16", f"largest slab {H}x{W} half {j}")
        del v
    assert_lse_close(to_f64(lse.reshape(N)[torch.from_numpy(rows).to(dev)])[None], want_lse, "bf16",
                     f"largest slab {H}x{W}")


@pytest.mark.parametrize("kd", [16, 32, 64, 128])
def test_psa_fused_fwd_degenerate_scores(kd):
    """Degenerate score rows: with the query channels zero every score is 0, so each output
    row is the mean of the V rows over all N keys and LSE = ln N (a closed form, and the oracle
    agrees); with every key row identical the same holds whatever the queries. Ties everywhere:
    the running max is set once and never moves."""
    dev = device()
    B, h, H, W = 2, 2, 13, 17
    N = H * W
    announce(f"psa_attention_fwd degenerate scores kd{kd}")
    qkv = I.make_qkv(B, h, kd, H, W, seed=60 + kd)
    g = qkv.clone().reshape(B, h, 4, kd, N)
    g[:, :, 0] = 0                                            # Q = 0
    zq = g.reshape(qkv.shape).contiguous()
    g = qkv.clone().reshape(B, h, 4, kd, N)
    g[:, :, 1] = g[:, :, 1, :, :1]                            # every key row equals the first
    same_k = g.reshape(qkv.shape).contiguous()
    for name, x in (("Q = 0", zq), ("identical keys", same_k)):
        out, _, lse = psa.psa_attention_fwd(x.to(dev), h, kd)
        v = to_f64(x).reshape(B * h, 4, kd, N)[:, 2:]          # [BH, 2, KD, N]
        want = np.broadcast_to(v.mean(axis=-1, keepdims=True), v.shape).reshape(B * h, 2 * kd, N)
        got = to_f64(out).reshape(B * h, 2 * kd, N)
        assert_attention_close(got, want, "bf16", f"{name}: out vs mean of V")
        if name == "Q = 0":
            assert np.abs(to_f64(lse) - np.log(N)).max() < 5e-3, "LSE is not ln N"
        want_out, _, want_lse = O.psa_forward(to_f64(x), B, h, kd, H, W)
        assert_attention_close(to_f64(out), want_out, "bf16", f"{name}: out vs oracle")
        assert_lse_close(to_f64(lse), want_lse, "bf16", f"{name}")
