"""Writes tests/golden/zipf_s.json: for every workload and non-zero maxvio
target, the Zipf bias strength s whose realised expert-level maxvio (oracle
route + count + stats on the workload's seeded logits) is closest to the
target. 40 bisection steps on [0, 20], ties to the smaller s.

Calls only the oracle. Run from the repository root:
    python tests/golden/make_zipf_s.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.workloads import WORKLOADS, key, skew_points  # noqa: E402


def realised(lg, bias, k, E, R):
    ids, _, _ = oracle.route(lg, bias, k)
    c = oracle.count(ids, E, R)
    return oracle.stats(ids, c["counts"], R)["maxvio_expert"]


def tune(name, target):
    w = WORKLOADS[name]
    T, E, k, R, seed = w["T"], w["E"], w["k"], w["R"], w["seed"]
    lg = synth.router_logits(T, E, seed)
    best = (abs(realised(lg, None, k, E, R) - target), 0.0)
    lo, hi = 0.0, 20.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        mv = realised(lg, synth.zipf_bias(E, mid, seed), k, E, R)
        cand = (abs(mv - target), mid)
        if cand < best:
            best = cand
        if mv < target:
            lo = mid
        else:
            hi = mid
    s = best[1]
    return dict(s=s, target=target, realised=realised(lg, synth.zipf_bias(E, s, seed), k, E, R),
                unbiased=realised(lg, None, k, E, R))


def main():
    out = {}
    for name, mv in skew_points():
        out[key(name, mv)] = tune(name, mv)
        print(key(name, mv), out[key(name, mv)], flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_s.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
