"""Choose the logit-offset amplitude A of the skewed-routing workload.

The workload adds c_e = A * r_e^(-1.1) to expert e's router logit, r being a
seeded ranking of the experts (Zipf with s = 1.1), and asks for the busiest
expert to receive about ten times the mean load T*k/E.  This script bisects A
on the workload's own inputs with the oracle's router (and nothing else) and
prints the value to put in moegen.SKEW_AMPLITUDE, with the load statistics.

Run:  python -m oracle.calibrate_skew
"""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import moegen
import oracle

TARGET = 10.0


def loads(cfg, x, wr, b, amp, pool):
    c = moegen.logit_bias(cfg, amplitude=amp)
    chunks = np.array_split(np.arange(cfg.T), 16)
    parts = pool.map(lambda idx: oracle.route(x[idx], wr, b, cfg.k, logit_bias=c)[0], chunks)
    ids = np.concatenate(list(parts))
    return np.bincount(ids.ravel(), minlength=cfg.E)


def main():
    cfg = moegen.CONFIGS[3]
    x, wr, b = moegen.x(cfg), moegen.router(cfg), moegen.sel_bias(cfg)
    mean = cfg.T * cfg.k / cfg.E
    lo, hi = 0.0, 8.0
    with ThreadPoolExecutor(max_workers=moegen.threads()) as pool:
        for _ in range(14):
            mid = 0.5 * (lo + hi)
            ratio = loads(cfg, x, wr, b, mid, pool).max() / mean
            print(f"A={mid:.4f} max/mean={ratio:.3f}", flush=True)
            if ratio < TARGET:
                lo = mid
            else:
                hi = mid
        amp = round(0.5 * (lo + hi), 3)
        cnt = loads(cfg, x, wr, b, amp, pool)
    print(f"A = {amp}: max {cnt.max()} (x{cnt.max() / mean:.2f} mean {mean:.1f}), idle {int((cnt == 0).sum())}, "
          f"<=2 tokens {int((cnt <= 2).sum())}, top loads {sorted(cnt)[-4:][::-1]}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
