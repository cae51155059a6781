"""Write the oracle's expected results for the full-size decode stacks.

Stack: 60 layers x 512 experts, hidden 4096, inter 1024, group 64, top-4, pre-norm with
eps 1e-6 (60 layers and 512 experts with 4 active per token: tr.news.hada.io 'Model
mimarisi'; hidden 4096: same section), seed 0, experts 4-bit or 2-bit. Tokens are the
generator's N(0,1) draws 0, 1, 2, ...; a draw is kept when the oracle's top-k margin is
at least 1e-3 at every layer, so that the selected experts are decided far from any tie.
For each kept draw the file stores the draw index, the experts and weights per layer, the
margins and the output h after the last layer (fp64).

Calls only the oracle and the input generator. Usage:
    python tests/golden/make_stack_golden.py --bits 4 --tokens 4   (also --bits 2, --bits 3)
"""
import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

L, E, H, I, K, EPS, SEED = 60, 512, 4096, 1024, 4, 1e-6, 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--bits", type=int, default=4)
    ap.add_argument("--tokens", type=int, default=4)
    ap.add_argument("--max-draws", type=int, default=200)
    args = ap.parse_args()
    routers = [synth.router(SEED, l, E, H) for l in range(L)]
    prov = synth.Provider(SEED, H, I, args.bits)
    kept = dict(draw=[], idx=[], w=[], margins=[], out=[])
    t0 = time.time()
    for d in range(args.max_draws):
        x = synth.token(SEED, d, H)
        r = oracle.stack(prov, routers, x, I, K, args.bits, 64, EPS, stop_margin=1e-3, keep_all=False)
        ok = r["layers_done"] == L and np.min(r["margins"]) >= 1e-3
        print(f"draw {d}: layers {r['layers_done']} min margin {np.nanmin(r['margins']):.2e} "
              f"{'kept' if ok else 'skipped'} ({time.time() - t0:.0f}s)", flush=True)
        if ok:
            kept["draw"].append(d)
            kept["idx"].append(r["idx"])
            kept["w"].append(r["w"])
            kept["margins"].append(r["margins"])
            kept["out"].append(r["out"])
            if len(kept["draw"]) == args.tokens:
                break
    path = os.path.join(HERE, f"stack_full_{args.bits}bit.npz")
    np.savez(path, draw=np.array(kept["draw"], dtype=np.int64), idx=np.array(kept["idx"], dtype=np.int32),
             w=np.array(kept["w"]), margins=np.array(kept["margins"]), out=np.array(kept["out"]),
             shape=np.array([L, E, H, I, K, args.bits, SEED]))
    print("wrote", path)


if __name__ == "__main__":
    main()
