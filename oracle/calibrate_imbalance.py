"""Choose the Zipf router-bias scale alpha of an imbalanced workload.

Uses only the oracle's router: logits without bias once, then for each trial
alpha the fp32 bias add and the top-k selection, bisecting alpha until the
busiest expert holds 8x the mean number of routed rows (T*k/E). Prints the
value to store in mixture_experts_layer_stable_amd.inputs.ZIPF_ALPHA.

    python -m oracle.calibrate_imbalance imbalanced_bf16
"""
import sys

import numpy as np

from mixture_experts_layer_stable_amd import inputs
from oracle import moe

TARGET = 8.0


def imbalance(z0, bias, k, E):
    z = z0 + bias[None, :]                 # float32 + float32: the router's one bias add
    idx = moe.select_topk(z, k)
    counts = np.bincount(idx.ravel(), minlength=E)
    return counts.max() / (idx.size / E), int((counts == 0).sum())


def calibrate(name):
    w = inputs.WORKLOADS[name]
    x = inputs.make_x(w).float().numpy()
    wr = inputs.make_wr(w).float().numpy()
    z0 = moe.router_logits(x, wr, None)
    lo, hi = 0.0, 8.0
    for _ in range(24):
        mid = 0.5 * (lo + hi)
        r, _ = imbalance(z0, inputs.make_bias(w, mid).numpy(), w.k, w.E)
        if r < TARGET:
            lo = mid
        else:
            hi = mid
    alpha = round(0.5 * (lo + hi), 4)
    r, zeros = imbalance(z0, inputs.make_bias(w, alpha).numpy(), w.k, w.E)
    print("%s: alpha=%.4f  max/mean=%.3f  zero-token experts=%d" % (name, alpha, r, zeros))
    return alpha


if __name__ == "__main__":
    for n in sys.argv[1:]:
        calibrate(n)
