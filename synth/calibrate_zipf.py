"""Find the Zipf router-bias scale beta of the 'qwen36_a3b_zipf' recipe.

Bisection on beta so that the seed-0, T=32 draw, routed by the CPU oracle, leaves
40% of the 256 experts untouched.  Uses only the generator and the oracle; prints the
beta to copy into configs.ZIPF_BETA and the realised untouched fraction.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
from synth import configs  # noqa: E402


def untouched(beta, T=32, seed=0):
    cfg = configs.with_shape(configs.CONFIGS["qwen36_a3b_zipf"], zipf_beta=beta)
    L = configs.make_layer(cfg, seed=seed, with_experts=False)
    x = configs.make_tokens(cfg, T, seed=seed)
    lg = oracle.router_logits(x, L["router_w"], L["router_b"]).astype(np.float32)
    ids, _ = oracle.route_topk(lg, cfg.k)
    return 1.0 - len(np.unique(ids)) / cfg.E


def main(target=0.40):
    lo, hi = 0.0, 2.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if untouched(mid) < target:
            lo = mid
        else:
            hi = mid
    beta = round(hi, 4)
    print(f"beta={beta} untouched={untouched(beta):.4f}")


if __name__ == "__main__":
    main()
