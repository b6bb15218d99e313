"""A wider run of the random sweeps in test_gpu_sweep.py, over a range of
seeds (router, dispatch and whole-layer configurations, each against the
oracle as in the collected tests). Not collected by pytest; run on a GPU as

    python tests/sweep_wide.py FIRST_SEED LAST_SEED

Each seed adds 60 router, 40 dispatch and 20 layer configurations.
"""
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), ".."))

import test_gpu_sweep as S  # noqa: E402


def main(first, last):
    n = 0
    t0 = time.time()
    for seed in range(first, last + 1):
        for i, c in enumerate(S._router_cfgs(60, seed=1000 + seed)):
            S.test_route_random_configs_bit_exact(i, c)
            n += 1
        for i, c in enumerate(S._dispatch_cfgs(40, seed=2000 + seed)):
            S.test_dispatch_random_configs_bit_exact(i, c)
            n += 1
        for w in S._layer_cfgs(20, seed=3000 + seed):
            w = dict(w, name=f"s{seed}_{w['name']}")
            S.test_layer_random_configs(w)
            n += 1
        print("seed", seed, "configurations passed so far:", n, f"({time.time() - t0:.1f} s)", flush=True)
    print("all passed:", n)


if __name__ == "__main__":
    main(int(sys.argv[1]), int(sys.argv[2]))
