"""Child process of test_threads_gpu.py: entry points called from several host threads at once.

Run in a fresh process so that the threads' first calls into the library (which fill its
per-device caches: CU count, occupancy, fa2_bwd_noalloc's scratch address) coincide. Each
thread issues its work on a torch stream of its own, three times over; afterwards the main
thread repeats every call on the default stream, and each thread's last results must equal
those bit for bit (every kernel here is deterministic: no atomics, fixed reduction orders).
Prints one line per case as it goes and "ALL OK" at the end; exits non-zero on a mismatch.
"""
import os
import sys
import threading

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import torch  # noqa: E402

import psa_inputs as I  # noqa: E402
import vision_transformer_attention_psapackqkv_amd as psa  # noqa: E402

DEV = torch.device("cuda:0")


def _psa_fwd(B, h, KD, H, W, seed):
    qkv = I.make_qkv(B, h, KD, H, W, seed=seed).to(DEV)

    def run():
        out, v, lse = psa.psa_attention_fwd(qkv, h, KD)
        return [out, v, lse]
    return f"psa_attention_fwd B{B}h{h}kd{KD}_{H}x{W}", run


def _fa2(BH, n, D, seed, dt="bf16"):
    q, k, v, do = (t.to(DEV) for t in I.make_attention_inputs(BH, n, n, D, dtype=dt, seed=seed,
                                                              with_dout=True))

    def run():
        o, lse = psa.fa2_fwd(q, k, v)
        return [o, lse, *psa.fa2_bwd(q, k, v, o, do, lse)]
    return f"fa2_fwd+fa2_bwd [{BH},{n},{D}] {dt}", run


def _fa2_noalloc(BH, n, D, seed):
    q, k, v, do = (t.to(DEV) for t in I.make_attention_inputs(BH, n, n, D, seed=seed, with_dout=True))

    def run():
        o, lse = psa.fa2_fwd(q, k, v)
        return [o, lse, *psa.fa2_bwd_noalloc(q, k, v, o, do, lse)]
    return f"fa2_bwd_noalloc [{BH},{n},{D}] (the only thread using the scratch)", run


def _psa_bwd(B, h, KD, H, W, seed):
    qkv = I.make_qkv(B, h, KD, H, W, seed=seed).to(DEV)
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn((B, 2 * h * KD, H, W), generator=g).to(torch.bfloat16).to(DEV)

    def run():
        out, _, lse = psa.psa_attention_fwd(qkv, h, KD, want_v=False)
        return [out, lse, psa.psa_attention_bwd(qkv, out, lse, dout, h, KD)]
    return f"psa_attention_fwd+bwd B{B}h{h}kd{KD}_{H}x{W}", run


def _layout(B, h, KD, H, W, seed, dt):
    qkv = I.make_qkv(B, h, KD, H, W, dtype=dt, seed=seed).to(DEV)

    def run():
        packed = psa.psa_pack_qkv(qkv, h, KD)
        v = psa.psa_extract_v(packed, B, h, KD, H, W)
        merged = psa.psa_merge_attn(packed[:2].contiguous(), B, h, KD, H, W)
        return [packed, v, merged]
    return f"pack/extract/merge B{B}h{h}kd{KD}_{H}x{W} {dt}", run


CASES = [
    _psa_fwd(4, 8, 64, 40, 40, 11),
    _psa_fwd(2, 2, 128, 20, 20, 12),
    _psa_fwd(8, 4, 32, 20, 20, 13),
    _psa_fwd(2, 4, 16, 24, 24, 14),
    _fa2(16, 700, 64, 15),
    _fa2(4, 300, 128, 16, dt="f32"),
    _fa2_noalloc(8, 500, 32, 17),
    _psa_bwd(2, 2, 32, 16, 16, 18),
    _layout(4, 8, 64, 40, 40, 19, "bf16"),
    _layout(2, 2, 32, 9, 13, 20, "f32"),
]


def _same(a, b):
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def main():
    torch.cuda.synchronize()
    results = [None] * len(CASES)
    errors = []
    start = threading.Barrier(len(CASES))

    def worker(i):
        try:
            s = torch.cuda.Stream(DEV)
            with torch.cuda.stream(s):
                start.wait()
                for _ in range(3):
                    res = CASES[i][1]()
            s.synchronize()
            results[i] = res
        except Exception as e:  # reported below, with the case's name
            errors.append(f"{CASES[i][0]}: {type(e).__name__}: {e}")

    print(f"[threads] {len(CASES)} host threads, one stream each", flush=True)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    if errors:
        print("\n".join(errors), flush=True)
        return 1
    bad = 0
    for (name, run), got in zip(CASES, results):
        want = run()
        torch.cuda.synchronize()
        ok = len(got) == len(want) and all(_same(a, b) for a, b in zip(got, want))
        print(f"[threads] {name}: {'same bits' if ok else 'DIFFERS'}", flush=True)
        bad += not ok
    if bad:
        return 1
    print("ALL OK", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
