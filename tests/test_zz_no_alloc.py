"""fa2_bwd_noalloc (the FA2 backward that allocates nothing: -Delta lives in the library's own
device scratch) against fa2_bwd with a caller workspace, through the C ABI, on two calls in a
row, the second smaller: the results must be bit-identical (same kernels, same inputs)."""
import numpy as np
import pytest
import torch

import psa_inputs as I
import vision_transformer_attention_psapackqkv_amd as psa
from tests.gpu_helpers import announce, bits, device

pytestmark = pytest.mark.gpu


def test_noalloc_matches_fa2_bwd_on_two_calls():
    dev = device()
    # First a large call, then a smaller one: the scratch keeps the first call's -Delta rows
    # beyond the second's, which the second must neither need nor read.
    for BH, n_q, n_k, D in ((32, 1600, 1600, 64), (6, 130, 200, 32)):
        announce(f"fa2_bwd_noalloc BH={BH} n_q={n_q} n_k={n_k} D={D}")
        q, k, v, do = (t.to(dev) for t in I.make_attention_inputs(BH, n_q, n_k, D, dtype="bf16",
                                                                  seed=BH + n_q + D, with_dout=True))
        o, lse = psa.fa2_fwd(q, k, v)
        want = psa.fa2_bwd(q, k, v, o, do, lse)
        outs = tuple(torch.full_like(t, float("nan")) for t in want)
        got = psa.fa2_bwd_noalloc(q, k, v, o, do, lse, dq=outs[0], dk=outs[1], dv=outs[2])
        torch.cuda.synchronize()
        assert all(g is t for g, t in zip(got, outs))
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert np.array_equal(bits(g), bits(w)), f"{name} differs from fa2_bwd"


def test_noalloc_rejects_more_rows_than_its_scratch():
    dev = device()
    BH, n = 2, (16 << 20) // 8 + 8
    q = torch.zeros((BH, n, 16), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((BH, n), dtype=torch.float32, device=dev)
    kv = torch.zeros((BH, 8, 16), dtype=torch.bfloat16, device=dev)
    with pytest.raises(psa.PsaError, match="scratch"):
        psa.fa2_bwd_noalloc(q, kv, kv, q, q, lse)
