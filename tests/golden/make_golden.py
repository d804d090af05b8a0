"""Writes tests/golden/c1_oracle.json: the fp64 oracle's outputs on the tiny
Mamba-2 workload C1 (N=2, H=4, d_k=16, d_v=32, W=4, r=4, T=16, fp32 inputs).

A regression fixture only: it records what the oracle computes today so that an
unintended change to the oracle's arithmetic shows up as a test failure. It is
not an independent pin (tests/oracle_pins.py holds those). Every value comes
from oracle/ alone:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def c1_problem():
    cfg = workloads.C1
    U = cfg.units
    S0 = workloads.initial_state(cfg).reshape(U, cfg.d_k, cfg.d_v).astype(np.float64)
    B = workloads.basis(cfg)[np.arange(U) % cfg.heads].astype(np.float64)
    steps = [workloads.step_inputs(cfg, t) for t in range(cfg.steps)]
    f = lambda x, e: x.reshape((U,) + ((e,) if e else ())).astype(np.float64)
    q = np.stack([f(s.q, cfg.d_k) for s in steps])
    k = np.stack([f(s.k, cfg.d_k) for s in steps])
    v = np.stack([f(s.v, cfg.d_v) for s in steps])
    dc = np.stack([f(s.decay, 0) for s in steps])
    return cfg, S0, B, q, k, v, dc


def main():
    cfg, S0, B, q, k, v, dc = c1_problem()
    out = oracle.run(cfg.rule, S0, B, q, k, v, dc, None, cfg.window, threads=1)
    fixture = {
        "workload": cfg.description,
        "made_by": "tests/golden/make_golden.py (oracle/ only)",
        # per (step, unit) output norms, and full vectors at two steps for units 0 and 7
        "y_exact_norms": np.linalg.norm(out["y_exact"], axis=-1).tolist(),
        "y_sketch_norms": np.linalg.norm(out["y_sketch"], axis=-1).tolist(),
        "y_exact_t3_t15_u0_u7": out["y_exact"][[3, 15]][:, [0, 7]].tolist(),
        "y_sketch_t3_t15_u0_u7": out["y_sketch"][[3, 15]][:, [0, 7]].tolist(),
        "S_win_frobenius": np.linalg.norm(out["S_win"].reshape(out["S_win"].shape[0], -1), axis=1).tolist(),
        "Sk_last_u0": out["Sk"][-1][0].tolist(),
    }
    with open(os.path.join(HERE, "c1_oracle.json"), "w") as fh:
        json.dump(fixture, fh)


if __name__ == "__main__":
    main()
