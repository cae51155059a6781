"""Write the oracle's expected results for the batched workload: 64 tokens through one
512-expert layer (hidden 4096, inter 1024, group 64, top-4, no pre-norm, seed 0), 4-bit.

Tokens are planted: expert popularity Zipf(1.1), 4 distinct experts per token pulled
through the real router (x = z + sum_j gamma_j r_e_j / |r_e_j|, gamma = 8, 7, 6, 5; see
synth.planted_token). A draw is kept when the oracle's winners are the planted experts
with top-k margin at least 1e-3. For the kept draws the file stores the draw indices, the
experts and weights, the margins and the O7 (bf16 contract) output of the layer (fp64).

Calls only the oracle and the input generator. Usage:
    python tests/golden/make_batch_golden.py
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

E, H, I, K, BITS, T, SEED, LAYER = 512, 4096, 1024, 4, 4, 64, 0, 0


def main():
    R = synth.router(SEED, LAYER, E, H)
    X, draws, d = [], [], 0
    while len(X) < T:
        x, ex = synth.planted_token(SEED, d, R, K)
        idx, _, _, m = oracle.route(R, x.astype(np.float64), K)
        if set(idx.tolist()) == set(ex.tolist()) and m >= 1e-3:
            X.append(x)
            draws.append(d)
        d += 1
    X = np.stack(X)
    t0 = time.time()
    prov = synth.Provider(SEED, H, I, BITS)
    r = oracle.layer_bf16(prov, LAYER, R, X, I, K, BITS, 64)
    print(f"{T} tokens from {d} draws, {len(set(r['idx'].ravel().tolist()))} distinct experts, "
          f"oracle {time.time() - t0:.1f}s")
    path = os.path.join(HERE, "batch64_4bit.npz")
    np.savez(path, draw=np.array(draws, dtype=np.int64), idx=r["idx"].astype(np.int32), w=r["w"],
             margins=r["margins"], out=r["out"], shape=np.array([E, H, I, K, BITS, T, SEED, LAYER]))
    print("wrote", path)


if __name__ == "__main__":
    main()
