"""The CPU oracle against its pins, and planted mistakes that the pins must catch.

Each mutant below is a copy of ``oracle/oracle.c`` with one plausible mistake
planted in it, compiled into a temporary library on the CPU. The real oracle
must pass every pin; every mutant must fail at least one.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the oracle")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# (name, text in oracle.c, replacement)
MUTANTS = [
    ("gdn_projection_sign", "m = decay[0] * (eye - beta * k[i] * k[j]);",
     "m = decay[0] * (eye + beta * k[i] * k[j]);"),
    ("gdn_gate_dropped", "m = decay[0] * (eye - beta * k[i] * k[j]);",
     "m = (eye - beta * k[i] * k[j]);"),
    ("kda_decay_after_projection", "m = (eye - beta * k[i] * k[j]) * decay[j];",
     "m = decay[i] * (eye - beta * k[i] * k[j]);"),
    ("mamba2_decay_dropped", "m = decay[0] * eye;", "m = eye;"),
    ("write_weight_dropped", "return rule == ORACLE_MAMBA2 ? 1.0 : beta;", "return 1.0;"),
    ("write_transposed_index", "(v ? w * k[i] * v[j] : 0.0)", "(v ? w * k[j % dk] * v[i % ncols] : 0.0)"),
    ("carry_back_not_transposed", "transpose_times(dk, dk, A, qv, qt);", "matmul(dk, dk, 1, A, qv, qt);"),
    ("coefficients_use_raw_query", "acc += Bu[(size_t)m * dk + i] * qt[i];",
     "acc += Bu[(size_t)m * dk + i] * qv[i];"),
    ("sketch_missing_intra", "y_sketch[tu * dv + j] = y2[j] + y1[j];", "y_sketch[tu * dv + j] = y2[j];"),
    ("window_product_reversed", "apply_token(dk, dk, M, A, tmp, w, kv, NULL); /* A <- M A */",
     "matmul(dk, dk, dk, A, M, tmp); memcpy(A, tmp, sizeof(double) * sz_a);"),
    ("intra_not_reset", "for (size_t i = 0; i < sz_s; ++i) R[i] = 0.0;\n          tau = 0;",
     "tau = 0;"),
    ("refresh_from_stale_state", "memcpy(Swin, S, sizeof(double) * sz_s);\n          matmul(r, dk, dv, Bu, Swin, Sk);",
     "matmul(r, dk, dv, Bu, Swin, Sk);\n          memcpy(Swin, S, sizeof(double) * sz_s);"),
    ("exact_read_before_update", "if (y_exact) transpose_times(dk, dv, S, qv, y_exact + tu * dv);",
     "if (y_exact) transpose_times(dk, dv, Swin, qv, y_exact + tu * dv);"),
    ("bf16_ties_away_from_zero", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
     "if (dropped >= 0x8000u) kept += 1u;"),
    ("bf16_truncates", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
     "(void)dropped;"),
    ("carried_query_not_recorded", "if (qt_out) memcpy(qt_out + tu * dk, qt, sizeof(double) * dk);",
     "if (qt_out) memcpy(qt_out + tu * dk, qv, sizeof(double) * dk);"),
    ("bf16_window_refresh_not_rounded",
     "matmul(r, dk, dv, Bu, Swin, Sk);\n          if (sketch_bf16) round_sketch(sz_k, Sk);",
     "matmul(r, dk, dv, Bu, Swin, Sk);"),
]


def test_mutants_listed_apply_once():
    src = open(oracle.SOURCE).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, f"mutant {name}: pattern found {src.count(old)} times"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1
    mutant = tmp_path / f"oracle_{name}.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / f"liboracle_{name}.so"
    oracle.build(out=str(so), source=str(mutant))
    L = oracle.lib(str(so))
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(L)
        except AssertionError as e:
            failures.append(f"{pin.__name__}: {e}")
    assert failures, f"planted mistake {name!r} passed every pin"


def test_oracle_reproduces_c1_fixture(oracle_lib):
    """Regression: the oracle still computes what tests/golden/c1_oracle.json recorded."""
    import json
    import os
    from tests.golden.make_golden import c1_problem
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "c1_oracle.json")))
    cfg, S0, B, q, k, v, dc = c1_problem()
    out = oracle.run(cfg.rule, S0, B, q, k, v, dc, None, cfg.window, _lib_override=oracle_lib)
    sel = lambda y: y[[3, 15]][:, [0, 7]]
    np.testing.assert_allclose(np.linalg.norm(out["y_exact"], axis=-1), fx["y_exact_norms"], rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(out["y_sketch"], axis=-1), fx["y_sketch_norms"], rtol=1e-12)
    np.testing.assert_allclose(sel(out["y_exact"]), fx["y_exact_t3_t15_u0_u7"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sel(out["y_sketch"]), fx["y_sketch_t3_t15_u0_u7"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["Sk"][-1][0], fx["Sk_last_u0"], rtol=1e-12, atol=1e-15)
    fro = np.linalg.norm(out["S_win"].reshape(out["S_win"].shape[0], -1), axis=1)
    np.testing.assert_allclose(fro, fx["S_win_frobenius"], rtol=1e-12)


# Planted mistakes in the basis fit (oracle.fit_basis, numpy): each copy of its source
# with one change must fail at least one of the fit pins.
FIT_MUTANTS = [
    ("fit_centred", "M = X[h].T @ X[h] / S",
     "M = (X[h] - X[h].mean(0)).T @ (X[h] - X[h].mean(0)) / S"),
    ("fit_not_normalised", "M = X[h].T @ X[h] / S", "M = X[h].T @ X[h]"),
    ("fit_ascending", 'order = np.argsort(-w, kind="stable")', 'order = np.argsort(w, kind="stable")'),
    ("fit_rows_of_V", "v = V[:, order[m]]", "v = V[order[m], :]"),
    ("fit_no_sign_rule", "out[h, m] = v if v[big] > 0 else -v", "out[h, m] = v"),
    ("fit_sign_by_first_entry", "big = int(np.argmax(np.abs(v)))", "big = 0"),
]


def _mutated_fit(old, new):
    import inspect
    src = inspect.getsource(oracle.fit_basis)
    assert src.count(old) == 1, f"pattern found {src.count(old)} times"
    ns = dict(oracle.__dict__)
    exec(src.replace(old, new), ns)
    return ns["fit_basis"]


@pytest.mark.parametrize("name,old,new", FIT_MUTANTS, ids=[m[0] for m in FIT_MUTANTS])
def test_planted_fit_mistake_is_caught(name, old, new):
    fit = _mutated_fit(old, new)
    failures = []
    for pin in oracle_pins.FIT_PINS:
        try:
            pin(None, fit=fit)
        except AssertionError as e:
            failures.append(f"{pin.__name__}: {e}")
    assert failures, f"planted mistake {name!r} passed every fit pin"
