"""The algorithmic byte counts behind bench.py's roofline, checked on the CPU against the
per-unit formulas written out here:
  update + refresh:  8 d_k d_v (S in and out) + s_sk r d_v (sketch out) + W tok (the window)
  sketch step:       s_sk r d_v + d_k s_in (q) + tau_mean tok (buffered tokens, the current
                     one included) + tok (the current token written) + 4 d_v (y)
with tok = (d_k + d_v) s_in + g, g = 4 (Mamba-2), 8 (GDN) or 4 d_k + 4 (KDA), and
tau_mean = (W + 1) / 2."""
import importlib.util
import os

import pytest

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(HERE, "..", "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def expected(cfg, s_sk=4):
    s_in = 2 if cfg.in_dtype == "bf16" else 4
    g = {"mamba2": 4, "gdn": 8, "kda": 4 * cfg.d_k + 4}[cfg.rule]
    tok = (cfg.d_k + cfg.d_v) * s_in + g
    update = 8 * cfg.d_k * cfg.d_v + s_sk * cfg.rank * cfg.d_v + cfg.window * tok
    step = (s_sk * cfg.rank * cfg.d_v + cfg.d_k * s_in + (cfg.window + 1) / 2 * tok + tok
            + 4 * cfg.d_v)
    return update, step


CASES = [workloads.get(n) for n in ("c1", "c2", "c3", "c4")] + \
        [workloads.c5(r, w) for r in (4, 8, 16, 32) for w in (4, 8, 16)]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("s_sk", [4, 2])
def test_byte_model(bench, cfg, s_sk):
    m = bench.bytes_model(cfg, s_sk)
    update, step = expected(cfg, s_sk)
    assert m["update"] == update
    assert m["sketch_step"] == pytest.approx(step)
    assert m["state_bytes_full"] == 4 * cfg.d_k * cfg.d_v
    assert m["state_bytes_sketch"] == s_sk * cfg.rank * cfg.d_v


def test_gdn_workload_update_bytes(bench):
    """GDN 128x128, W = 8, r = 8, bf16: 131072 + 4096 + 8 * 520 bytes per unit, and 8192 units
    per launch for the roofline's algorithmic bytes."""
    cfg = workloads.C3
    assert bench.bytes_model(cfg)["update"] == 139_328
    assert bench.bytes_model(cfg)["update"] * cfg.units == 1_141_374_976


@pytest.mark.parametrize("steps,warmup,want", [(20, 5, (24, 8)), (64, 16, (64, 16)),
                                               (1, 0, (8, 0)), (0, 0, (8, 0)), (9, 17, (16, 24))])
def test_step_rounding(bench, steps, warmup, want):
    """Any --steps / --warmup is accepted: both are rounded up to whole windows (W = 8 here),
    with at least one timed window, so every window's update + refresh is inside the region
    it belongs to and the timed count is what ms_per_step describes."""
    a = bench.parse_args(["--gpus", "1", "--steps", str(steps), "--warmup", str(warmup)])
    assert (a.steps, a.warmup) == (steps, warmup)
    got = bench.plan_steps(a.steps, a.warmup, workloads.C3.window)
    assert got == want
    assert got[0] % 8 == 0 and got[1] % 8 == 0 and got[0] >= steps and got[1] >= warmup


def test_step_rounding_sweep_windows(bench):
    """The sweep rounds to the largest window (16), a multiple of every sweep window."""
    steps, warmup = bench.plan_steps(20, 5, max(workloads.C5_WINDOWS))
    assert (steps, warmup) == (32, 16)
    assert all(steps % w == 0 and warmup % w == 0 for w in workloads.C5_WINDOWS)


def test_error_summary(bench):
    """The approximation-error record: the global Frobenius ratio over all outputs and the
    per-vector distribution, from per-vector squared norms."""
    num = [[1.0, 4.0], [0.0, 9.0]]     # ||dy||^2 per (step, unit)
    den = [[1.0, 16.0], [4.0, 9.0]]    # ||y_exact||^2
    s = bench.error_summary(num, den)
    assert s["frobenius"] == pytest.approx((14.0 / 30.0) ** 0.5)
    assert s["max"] == pytest.approx(1.0)
    assert s["mean"] == pytest.approx((1.0 + 0.5 + 0.0 + 1.0) / 4)
    assert s["vectors"] == 4


def test_bench_rejects_only_gpu_counts(bench, capsys):
    """--gpus above 1 is the only argument the bench refuses, with a message."""
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
