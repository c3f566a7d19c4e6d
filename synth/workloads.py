"""The layer shapes exercised by tests and the benchmark, with their seeds and
router-skew settings. Data only.

Shapes (tokens T, hidden H, routed experts E, top-k, SwiGLU width F, virtual
ranks R, replica slots S):
  tiny      fp32  T=16    H=64   E=8   k=2 F=128   R=4  S=2  (and the 16-token
                  hotspot fixture's exact expert pairs)
  mixtral   bf16  T=2048  H=4096 E=8   k=2 F=14336 R=8  S=1  maxvio 0.2
  a3b       bf16  T=4096  H=2048 E=128 k=8 F=768   R=16 S=8  maxvio 0, 0.2, 1
  dsv3      bf16  T=8192  H=7168 E=256 k=8 F=2048  R=32 S=8  + one shared expert
                  of width 2048; maxvio 20 and 0
  decodeT   bf16  T in {64, 256, 1024} H=4096 E=128 k=8 F=1536 R=16 S=3;
                  maxvio 1 and 20 (20 exceeds E/k - 1 = 15, the most any
                  router with distinct top-k can reach here, so the run lands
                  at 15); capacity figures at factor 1.25.

Router skew: maxvio 0 uses the exactly-even fixed-count mode; any other
target uses N(0,1) logits plus the Zipf-shaped bias -s*ln(1+pi(e)), with s
read from tests/golden/zipf_s.json (chosen there by bisection so that the
realised expert maxvio is as close to the target as the draw allows).
"""
from __future__ import annotations

import json
import os

from . import even_logits, fixture_logits, router_logits, zipf_bias

_S_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests",
                       "golden", "zipf_s.json")

WORKLOADS = {
    "tiny": dict(T=16, H=64, E=8, k=2, F=128, R=4, S=2, dtype="f32", seed=1, maxvio=[None]),
    "mixtral": dict(T=2048, H=4096, E=8, k=2, F=14336, R=8, S=1, dtype="bf16", seed=2,
                    maxvio=[0.2]),
    "a3b": dict(T=4096, H=2048, E=128, k=8, F=768, R=16, S=8, dtype="bf16", seed=3,
                maxvio=[0, 0.2, 1]),
    "dsv3": dict(T=8192, H=7168, E=256, k=8, F=2048, R=32, S=8, dtype="bf16", seed=4,
                 shared_F=2048, maxvio=[20, 0]),
    "decode64": dict(T=64, H=4096, E=128, k=8, F=1536, R=16, S=3, dtype="bf16", seed=5,
                     maxvio=[1, 20], capacity_factor=1.25),
    "decode256": dict(T=256, H=4096, E=128, k=8, F=1536, R=16, S=3, dtype="bf16", seed=5,
                      maxvio=[1, 20], capacity_factor=1.25),
    "decode1024": dict(T=1024, H=4096, E=128, k=8, F=1536, R=16, S=3, dtype="bf16", seed=5,
                       maxvio=[1, 20], capacity_factor=1.25),
}


def key(name: str, maxvio) -> str:
    return f"{name}@{maxvio:g}"


def zipf_s(name: str, maxvio) -> float:
    with open(_S_FILE) as f:
        table = json.load(f)
    return float(table[key(name, maxvio)]["s"])


def logits_and_bias(name: str, maxvio):
    """(logits [T,E] float32, bias [E] float32 or None) for a workload at a skew
    target; maxvio None means plain N(0,1) logits and no bias."""
    w = WORKLOADS[name]
    T, E, k, seed = w["T"], w["E"], w["k"], w["seed"]
    if maxvio is None:
        return router_logits(T, E, seed), None
    if maxvio == 0:
        return even_logits(T, E, k, seed), None
    return router_logits(T, E, seed), zipf_bias(E, zipf_s(name, maxvio), seed)


def fixture():
    """The 16-token hotspot fixture's logits (E = 8, top-2)."""
    return fixture_logits(), None


def skew_points():
    for name, w in WORKLOADS.items():
        for mv in w["maxvio"]:
            if mv:
                yield name, mv
