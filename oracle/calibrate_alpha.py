"""Bisection of the heavy-hitter strength alpha of the top-p decode workloads.

Finds alpha such that the oracle's top-p(0.9) support of group 0 holds 10% of
the context (before the sink/window union), on CPU-drawn inputs:

  * the 64K decode workload (32 query / 4 key-value heads, 1% heavy hitters);
  * a 64K row shaped like the batched workload (32 / 8 heads, 1% heavy hitters).

The frozen results live in synth/gen.py (ALPHA_DECODE64K, ALPHA_BATCHED).
Run:  python -m oracle.calibrate_alpha
"""

import sys

import numpy as np
import torch

import oracle as O
import synth


def budget(inp, p=0.9, g=0):
    hs = inp.heads(g)
    q = inp.q[0, hs].double().numpy()
    wq = inp.w_q[hs].double().numpy()
    K = inp.seq_keys(0, g).double().numpy()
    kt = O.round_to_bf16(O.indexer_keys(K, inp.w_k[g].double().numpy()))
    x = O.token_scores(O.collapse_query(q, wq, inp.s_idx), kt)
    return len(O.select_topp(x, p)) / K.shape[0]


def bisect(make, target=0.10, lo=0.0, hi=80.0, steps=24):
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        b = budget(make(mid))
        print(f"  alpha={mid:.4f} budget={b:.4f}", flush=True)
        if b > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def main():
    torch.set_num_threads(8)
    a64 = bisect(lambda a: synth.make_decode64k(device="cpu", alpha=a))
    print(f"ALPHA_DECODE64K = {a64:.3f}")
    ab = bisect(lambda a: synth.make_decode_custom(
        name="calib_batched", B=1, H_q=32, H_kv=8, d=128, seq_lens=[65536],
        dtype=torch.bfloat16, device="cpu", seed=0, cfg=5, hh_frac=0.01, alpha=a,
        tied=True))
    print(f"ALPHA_BATCHED = {ab:.3f}")


if __name__ == "__main__":
    sys.exit(main())
