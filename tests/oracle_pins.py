"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function takes a loaded oracle library and raises
``AssertionError`` when the oracle breaks the fact it checks. The facts are
hand-worked numbers, closed forms of the recurrences, algebraic invariants
of the method and brute force through a different route (chaining single
steps instead of the run's window bookkeeping). ``test_oracle_pins.py``
runs them on the real oracle and on deliberately broken copies of it, and
each broken copy must fail at least one pin.

Sources: readsearch.ai listing of arXiv 2609.33051 (SketchSSM), Abstract;
agihunt.info summary of SketchSSM, "Mechanism details" and "Error control".
"""
from __future__ import annotations

import numpy as np

import oracle

RULES = ("mamba2", "gdn", "kda")


# ----------------------------------------------------------------------------
# tiny seeded problems (shapes: see oracle.run)
# ----------------------------------------------------------------------------
def orthonormal_rows(rng, r, dk):
    qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    return np.ascontiguousarray(qm[:, :r].T)


def problem(rule, *, U=3, dk=6, dv=5, r=3, W=3, T=7, seed=0, beta_lo=0.1, beta_hi=0.9):
    rng = np.random.default_rng([0xC0DE, seed, RULES.index(rule)])
    S0 = rng.standard_normal((U, dk, dv)) * 0.3
    basis = np.stack([orthonormal_rows(rng, r, dk) for _ in range(U)])
    q = rng.standard_normal((T, U, dk))
    k = rng.standard_normal((T, U, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, U, dv))
    if rule == "kda":
        decay = rng.uniform(0.5, 1.0, size=(T, U, dk))
    else:
        decay = rng.uniform(0.5, 1.0, size=(T, U))
    beta = None if rule == "mamba2" else rng.uniform(beta_lo, beta_hi, size=(T, U))
    return dict(rule=rule, S0=S0, basis=basis, q=q, k=k, v=v, decay=decay, beta=beta, window=W)


def run(L, p, **kw):
    return oracle.run(p["rule"], p["S0"], p["basis"], p["q"], p["k"], p["v"], p["decay"],
                      p["beta"], p["window"], _lib_override=L, **kw)


def _beta(p, t, u):
    return 0.0 if p["beta"] is None else float(p["beta"][t, u])


def chain_steps(L, p, u, t0, t1, S, with_v=True):
    """Apply tokens t0..t1-1 of unit u to S by single steps (v = 0 if not with_v)."""
    X = S.copy()
    for t in range(t0, t1):
        v = p["v"][t, u] if with_v else np.zeros(X.shape[1])
        X = oracle.rule_step(p["rule"], X, p["k"][t, u], v, p["decay"][t, u], _beta(p, t, u),
                             _lib_override=L)
    return X


def close(a, b, tol=1e-10, what=""):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs diff {err:.3e} (scale {scale:.3e})"


# ----------------------------------------------------------------------------
# single-token rule
# ----------------------------------------------------------------------------
def pin_hand_worked_steps(L):
    """Two-dimensional steps worked out by hand (k = (0.6, 0.8), beta = 0.5).

    GDN, alpha = 0.5: M = 0.5 (I - 0.5 k k^T) = [[0.41, -0.12], [-0.12, 0.34]].
    KDA, alpha = (0.5, 0.25): M = (I - 0.5 k k^T) Diag(alpha) = [[0.41, -0.06], [-0.12, 0.17]].
    Mamba-2, a = 0.3: M = 0.3 I.
    With S = [[1, 2], [3, 4]] and v = (1, -1), the write b k v^T is
    [[0.3, -0.3], [0.4, -0.4]] for the delta rules (b = beta) and
    [[0.6, -0.6], [0.8, -0.8]] for Mamba-2 (b = 1).
    """
    k = np.array([0.6, 0.8])
    v = np.array([1.0, -1.0])
    S = np.array([[1.0, 2.0], [3.0, 4.0]])
    close(oracle.transition_matrix("gdn", k, 0.5, 0.5, _lib_override=L),
          [[0.41, -0.12], [-0.12, 0.34]], 1e-14, "GDN M")
    close(oracle.transition_matrix("kda", k, [0.5, 0.25], 0.5, _lib_override=L),
          [[0.41, -0.06], [-0.12, 0.17]], 1e-14, "KDA M")
    close(oracle.transition_matrix("mamba2", k, 0.3, 0.0, _lib_override=L),
          [[0.3, 0.0], [0.0, 0.3]], 1e-14, "Mamba-2 M")
    close(oracle.rule_step("gdn", S, k, v, 0.5, 0.5, _lib_override=L),
          [[0.35, 0.04], [1.30, 0.72]], 1e-14, "GDN step")
    close(oracle.rule_step("kda", S, k, v, [0.5, 0.25], 0.5, _lib_override=L),
          [[0.53, 0.28], [0.79, 0.04]], 1e-14, "KDA step")
    close(oracle.rule_step("mamba2", S, k, v, 0.3, 0.0, _lib_override=L),
          [[0.9, 0.0], [1.7, 0.4]], 1e-14, "Mamba-2 step")


def pin_delta_overwrite(L):
    """Delta rules at beta = 1 with a unit key store v exactly: k^T S_new = v^T."""
    rng = np.random.default_rng(11)
    for rule in ("gdn", "kda"):
        for _ in range(5):
            dk, dv = 7, 4
            S = rng.standard_normal((dk, dv))
            k = rng.standard_normal(dk)
            k /= np.linalg.norm(k)
            v = rng.standard_normal(dv)
            a = rng.uniform(0.3, 1.0, size=dk) if rule == "kda" else rng.uniform(0.3, 1.0)
            Sn = oracle.rule_step(rule, S, k, v, a, 1.0, _lib_override=L)
            close(k @ Sn, v, 1e-12, f"{rule} overwrite")


def pin_pure_decay(L):
    """beta = 0 leaves only the decay; Mamba-2 with k = 0 is a pure decay too."""
    rng = np.random.default_rng(12)
    dk, dv = 6, 3
    S = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    close(oracle.rule_step("gdn", S, k, v, 0.7, 0.0, _lib_override=L), 0.7 * S, 1e-14, "GDN decay")
    a = rng.uniform(0.2, 1.0, size=dk)
    close(oracle.rule_step("kda", S, k, v, a, 0.0, _lib_override=L), a[:, None] * S, 1e-14,
          "KDA decay is per key channel (rows)")
    close(oracle.rule_step("mamba2", S, np.zeros(dk), v, 0.7, 0.0, _lib_override=L), 0.7 * S,
          1e-14, "Mamba-2 decay")
    # Mamba-2 write is the plain outer product, whatever beta says
    close(oracle.rule_step("mamba2", S, k, v, 1.0, 0.25, _lib_override=L), S + np.outer(k, v),
          1e-14, "Mamba-2 write")


def pin_kda_uniform_is_gdn(L):
    """KDA with a gate vector alpha = a * 1 is GDN with scalar gate a (whole runs)."""
    p = problem("gdn", seed=3)
    pk = dict(p, rule="kda", decay=np.repeat(p["decay"][:, :, None], p["S0"].shape[1], axis=2))
    a, b = run(L, p), run(L, pk)
    for key in ("y_exact", "y_sketch", "y_replay", "S_win", "Sk"):
        close(b[key], a[key], 1e-12, f"KDA(uniform) vs GDN {key}")


def pin_mamba2_closed_form(L):
    """Mamba-2: S_t = (prod a) S_0 + sum_i (prod_{j>i} a_j) k_i v_i^T, y_t = S_t^T q_t."""
    p = problem("mamba2", U=2, dk=5, dv=4, r=2, W=4, T=9, seed=4)
    out = run(L, p)
    T, U = p["q"].shape[:2]
    for u in range(U):
        for t in range(T):
            a = p["decay"][: t + 1, u]
            S = np.prod(a) * p["S0"][u]
            for i in range(t + 1):
                S = S + np.prod(a[i + 1:]) * np.outer(p["k"][i, u], p["v"][i, u])
            close(out["y_exact"][t, u], S.T @ p["q"][t, u], 1e-11, "Mamba-2 y closed form")
            if (t + 1) % p["window"] == 0:
                close(out["S_win"][(t + 1) // p["window"], u], S, 1e-11, "Mamba-2 S closed form")


# ----------------------------------------------------------------------------
# window bookkeeping against chained single steps (brute force, another route)
# ----------------------------------------------------------------------------
def pin_window_states_and_refresh(L):
    """Window-start states equal chained single steps; each sketch is B S_win."""
    for rule in RULES:
        p = problem(rule, seed=5)
        out = run(L, p)
        W = p["window"]
        T, U = p["q"].shape[:2]
        for u in range(U):
            S = p["S0"][u]
            for w in range(T // W + 1):
                if w > 0:
                    S = chain_steps(L, p, u, (w - 1) * W, w * W, S)
                close(out["S_win"][w, u], S, 1e-12, f"{rule} S_win[{w}]")
                close(out["Sk"][w, u], p["basis"][u] @ S, 1e-12, f"{rule} Sk[{w}] = B S_win")


def _window_pieces(L, p, u, t):
    """(S_win, A, R) for token t of unit u, by chaining single steps.

    A is the linear response of the window's tokens (state = I, no writes);
    R is their response from a zero state with the writes.
    """
    W = p["window"]
    t0 = (t // W) * W
    dk, dv = p["S0"].shape[1:]
    S_win = chain_steps(L, p, u, 0, t0, p["S0"][u])
    A = chain_steps(L, p, u, t0, t + 1, np.eye(dk), with_v=False)
    R = chain_steps(L, p, u, t0, t + 1, np.zeros((dk, dv)))
    return S_win, A, R


def pin_decomposition(L):
    """S_t = A_t S_win + R_t; the run's A and R equal the linear responses."""
    for rule in RULES:
        p = problem(rule, U=2, seed=6)
        out = run(L, p, want_A=True, want_R=True)
        T, U = p["q"].shape[:2]
        for u in range(U):
            for t in range(T):
                S_win, A, R = _window_pieces(L, p, u, t)
                close(out["A"][t, u], A, 1e-12, f"{rule} A[{t}]")
                close(out["R"][t, u], R, 1e-12, f"{rule} R[{t}]")
                S_t = chain_steps(L, p, u, 0, t + 1, p["S0"][u])
                close(A @ S_win + R, S_t, 1e-12, f"{rule} decomposition at {t}")
                close(out["y_exact"][t, u], S_t.T @ p["q"][t, u], 1e-12, f"{rule} y_exact")
                close(out["y_replay"][t, u], out["y_exact"][t, u], 1e-12,
                      f"{rule} window-start read equals exact read")


def pin_error_identity(L):
    """y_exact - y_sketch = S_win^T (I - B^T B) A^T q, with A from the linear response."""
    for rule in RULES:
        p = problem(rule, U=2, dk=6, dv=4, r=2, seed=7)
        out = run(L, p)
        T, U = p["q"].shape[:2]
        for u in range(U):
            B = p["basis"][u]
            P_perp = np.eye(B.shape[1]) - B.T @ B
            for t in range(T):
                S_win, A, R = _window_pieces(L, p, u, t)
                qt = A.T @ p["q"][t, u]
                close(out["y_exact"][t, u] - out["y_sketch"][t, u], S_win.T @ (P_perp @ qt),
                      1e-11, f"{rule} error identity at {t}")
                close(out["y_sketch"][t, u], (B @ S_win).T @ (B @ qt) + R.T @ p["q"][t, u],
                      1e-11, f"{rule} sketch output at {t}")


# ----------------------------------------------------------------------------
# invariants of the method
# ----------------------------------------------------------------------------
def pin_full_basis_is_exact(L):
    """r = d_k: B = I, or any orthogonal B, gives the exact read."""
    rng = np.random.default_rng(13)
    for rule in RULES:
        p = problem(rule, dk=5, r=5, seed=8)
        U, dk = p["S0"].shape[:2]
        for B in (np.tile(np.eye(dk), (U, 1, 1)),
                  np.stack([orthonormal_rows(rng, dk, dk) for _ in range(U)])):
            out = run(L, dict(p, basis=B))
            close(out["y_sketch"], out["y_exact"], 1e-11, f"{rule} full-rank sketch is exact")


def pin_span_invariance(L):
    """Rotating the basis inside its span (B -> Q B, Q orthogonal r x r) changes no output."""
    rng = np.random.default_rng(14)
    for rule in RULES:
        p = problem(rule, seed=9)
        U, r = p["basis"].shape[:2]
        Q = np.stack([orthonormal_rows(rng, r, r) for _ in range(U)])
        a = run(L, p)
        b = run(L, dict(p, basis=np.einsum("umn,unk->umk", Q, p["basis"])))
        close(b["y_sketch"], a["y_sketch"], 1e-11, f"{rule} span invariance")


def pin_linearity_in_q(L):
    """Both reads are linear in the query."""
    rng = np.random.default_rng(15)
    for rule in RULES:
        p = problem(rule, seed=10)
        q2 = rng.standard_normal(p["q"].shape)
        a = run(L, p)
        b = run(L, dict(p, q=q2))
        c = run(L, dict(p, q=p["q"] - 2.5 * q2))
        for key in ("y_exact", "y_sketch"):
            close(c[key], a[key] - 2.5 * b[key], 1e-11, f"{rule} linearity {key}")


def pin_queries_do_not_touch_state(L):
    """Changing one query changes that step's outputs only; states and sketches stay."""
    for rule in RULES:
        p = problem(rule, seed=16)
        q = p["q"].copy()
        q[4] = -3.0 * q[4] + 1.0
        a = run(L, p)
        b = run(L, dict(p, q=q))
        for key in ("S_win", "Sk"):
            assert np.array_equal(a[key], b[key]), f"{rule}: query changed {key}"
        keep = [t for t in range(q.shape[0]) if t != 4]
        for key in ("y_exact", "y_sketch"):
            assert np.array_equal(a[key][keep], b[key][keep]), f"{rule}: query leaked into {key}"
            assert not np.allclose(a[key][4], b[key][4]), f"{rule}: query ignored in {key}"


def pin_mamba2_in_span_exact(L):
    """Mamba-2 carries q back by a scalar, so a query inside span(B) is read exactly."""
    rng = np.random.default_rng(17)
    p = problem("mamba2", seed=11)
    coef = rng.standard_normal(p["q"].shape[:2] + (p["basis"].shape[1],))
    q = np.einsum("tum,umk->tuk", coef, p["basis"])
    out = run(L, dict(p, q=q))
    close(out["y_sketch"], out["y_exact"], 1e-11, "Mamba-2 in-span exactness")


def pin_scalar_hand_case(L):
    """d_k = d_v = 1, W = 2, Mamba-2, worked by hand.

    S0 = 2; a = (0.5, 0.5, 0.25); k = (1, 2, 1); v = (3, 1, 4); q = (1, 1, 2).
    t1: S = 0.5*2 + 1*3 = 4, y = 4.  t2: S = 0.5*4 + 2*1 = 4, y = 4 (window ends, S_win = 4).
    t3: S = 0.25*4 + 1*4 = 5, y = 5*2 = 10. With d_k = 1 the sketch is exact.
    """
    p = dict(rule="mamba2", S0=np.array([[[2.0]]]), basis=np.array([[[1.0]]]),
             q=np.array([1.0, 1.0, 2.0]).reshape(3, 1, 1), k=np.array([1.0, 2.0, 1.0]).reshape(3, 1, 1),
             v=np.array([3.0, 1.0, 4.0]).reshape(3, 1, 1), decay=np.array([0.5, 0.5, 0.25]).reshape(3, 1),
             beta=None, window=2)
    out = run(L, p)
    close(out["y_exact"].ravel(), [4.0, 4.0, 10.0], 1e-15, "scalar y_exact")
    close(out["y_sketch"].ravel(), [4.0, 4.0, 10.0], 1e-15, "scalar y_sketch")
    close(out["S_win"].ravel(), [2.0, 4.0], 1e-15, "scalar S_win")


# ----------------------------------------------------------------------------
# bf16 sketch storage (an option: the pages leave the sketch's precision open)
# ----------------------------------------------------------------------------
def pin_bf16_rounding_cases(L):
    """Round to nearest bf16, ties to even, after rounding to fp32: values worked by hand.

    bf16 keeps 8 significant bits, so near 1 the spacing is 2^-7 and 1 + 2^-8 is
    exactly half way between 1 (pattern 0x3F80, even) and 1 + 2^-7 (0x3F81, odd).
    """
    f = lambda x: oracle.round_bf16(x, _lib_override=L)
    e = 2.0 ** -8
    cases = [
        (1.0, 1.0),
        (1 + e, 1.0),                     # tie, the even neighbour is 1
        (1 + 3 * e, 1 + 4 * e),           # tie between 0x3F81 (odd) and 0x3F82 (even)
        (1 + e + 2.0 ** -20, 1 + 2 * e),  # above half
        (1 + e - 2.0 ** -20, 1.0),        # below half
        (-(1 + 3 * e), -(1 + 4 * e)),     # sign symmetric
        (1 + e + 2.0 ** -30, 1.0),        # fp32 first: the 2^-30 is lost, then a tie
        ((2 - e) * 2.0 ** 127, np.inf),   # half way above the largest bf16: to infinity
        (3.0, 3.0), (0.0, 0.0),
    ]
    for x, want in cases:
        got = f(x)
        assert got == want, f"round_bf16({x!r}) = {got!r}, want {want!r}"
    assert np.copysign(1.0, f(-0.0)) == -1.0, "the sign of zero is kept"
    assert np.isnan(f(float("nan")))


def pin_bf16_rounding_matches_torch(L):
    """The rounding equals torch's fp32 -> bfloat16 conversion (round to nearest even) on
    random fp32 values and on values built to sit exactly on ties."""
    import torch
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-20, 20, 4000))).astype(np.float32)
    ties = (np.float32(1.0) + np.arange(1, 200, dtype=np.float32) * np.float32(2.0 ** -8))
    x = np.concatenate([x, ties, -ties]).astype(np.float64)
    want = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(v, _lib_override=L) for v in x])
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} values differ, e.g. {x[bad[0]]!r}: {got[bad[0]]!r} vs {want[bad[0]]!r}"


def pin_bf16_sketch_enters_only_the_sketch_read(L):
    """With a bf16 sketch every stored sketch (each window) is the fp32 sketch rounded
    (checked against torch's conversion); the exact reads do not change; and y_sketch
    moves by exactly (Sk_bf16 - Sk_f32)^T c with c = B A^T q from the same run."""
    import torch
    for rule in RULES:
        p = problem(rule, U=2, dk=6, dv=5, r=3, W=3, T=7, seed=5)
        a = run(L, p, want_A=True)
        b = run(L, p, want_A=True, sketch_bf16=True)
        want = torch.from_numpy(a["Sk"]).to(torch.float32).to(torch.bfloat16).to(torch.float64)
        assert np.array_equal(b["Sk"], want.numpy()), f"{rule}: stored sketch not rounded"
        assert not np.array_equal(a["Sk"], b["Sk"]), f"{rule}: rounding changed nothing"
        for key in ("y_exact", "y_replay", "S_win"):
            assert np.array_equal(a[key], b[key]), f"{rule}: {key} changed"
        T, U = p["q"].shape[:2]
        W = p["window"]
        for t in range(T):
            win = t // W
            for u in range(U):
                qt = a["A"][t, u].T @ p["q"][t, u]
                c = p["basis"][u] @ qt
                dy = (b["Sk"][win, u] - a["Sk"][win, u]).T @ c
                close(b["y_sketch"][t, u] - a["y_sketch"][t, u], dy, 1e-12,
                      f"{rule} t={t} u={u} y_sketch shift")


# ----------------------------------------------------------------------------
# least-squares coefficients (the alternative reading of "state-weighted")
# ----------------------------------------------------------------------------
def pin_ls_exact_for_rank_one_state(L):
    """A rank-1 window-start state S = u w^T has outputs along w only, and the sketch
    rows B S = (B u) w^T span w: the least-squares read is exact in that window, while
    the projection read c = B q~ is not (q~ is not in the span of B)."""
    for rule in RULES:
        p = problem(rule, U=2, dk=6, dv=5, r=2, W=4, T=4, seed=7)
        rng = np.random.default_rng(3)
        for u in range(2):
            p["S0"][u] = np.outer(rng.standard_normal(6), rng.standard_normal(5))
        out = run(L, p, want_ls=True)
        close(out["y_ls"], out["y_replay"], 1e-9, f"{rule} rank-1 LS read")
        err = np.abs(out["y_sketch"] - out["y_replay"]).max()
        assert err > 1e-3, f"{rule}: the projection read is unexpectedly exact ({err:.2e})"


def pin_ls_full_rank_is_exact(L):
    """r = d_k: the sketch rows span the state's row space, so the read is exact."""
    for rule in RULES:
        p = problem(rule, U=2, dk=5, dv=6, r=5, W=3, T=7, seed=8)
        out = run(L, p, want_ls=True)
        close(out["y_ls"], out["y_replay"], 1e-9, f"{rule} full-rank LS read")


def pin_ls_never_worse_than_projection(L):
    """Least squares minimises the read error over all c, so per step its error against
    the exact read is at most that of c = B q~."""
    for rule in RULES:
        p = problem(rule, U=3, dk=6, dv=5, r=2, W=3, T=7, seed=9)
        out = run(L, p, want_ls=True)
        e_ls = np.linalg.norm(out["y_ls"] - out["y_replay"], axis=-1)
        e_pr = np.linalg.norm(out["y_sketch"] - out["y_replay"], axis=-1)
        assert np.all(e_ls <= e_pr + 1e-12), f"{rule}: LS error above the projection's"
        assert np.any(e_ls < e_pr - 1e-6), f"{rule}: LS never better than the projection"


def pin_ls_zero_state(L):
    """S_win = 0: the sketch is zero, every c gives Sk^T c = 0 and the read is the
    window term R^T q alone (the rank-deficient case takes the smallest c)."""
    for rule in RULES:
        p = problem(rule, U=2, dk=4, dv=3, r=2, W=3, T=3, seed=10)
        p["S0"][:] = 0.0
        out = run(L, p, want_ls=True)
        close(out["y_ls"], out["y_replay"], 1e-12, f"{rule} zero state")
        close(out["y_ls"], out["y_sketch"], 1e-12, f"{rule} zero state vs projection")


# ----------------------------------------------------------------------------
# the offline basis fit (oracle.fit_basis, numpy): top-r eigenvectors of the
# uncentred second moment of sampled queries. Each pin takes the fit function so
# that test_oracle_pins.py can run the same pins on copies with planted mistakes.
# ----------------------------------------------------------------------------
def _sign_rule(rows):
    """Rows signed so that the entry of largest magnitude (first on a tie) is positive."""
    out = np.array(rows, dtype=np.float64)
    for m in range(out.shape[0]):
        if out[m, int(np.argmax(np.abs(out[m])))] < 0:
            out[m] = -out[m]
    return out


def pin_fit_closed_form(L, fit=oracle.fit_basis):
    """Samples X = sqrt(S) Z diag(sig) U^T with Z^T Z = I have second moment
    X^T X / S = U diag(sig^2) U^T: the fit must return the columns of U ordered by
    decreasing sig (signed by the rule) and the eigenvalues sig^2."""
    rng = np.random.default_rng(11)
    H, S, dk, r = 2, 40, 6, 4
    X = np.empty((H, S, dk))
    want_rows, want_lam = [], []
    for h in range(H):
        Z, _ = np.linalg.qr(rng.standard_normal((S, dk)))
        U, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        sig = rng.permutation(np.array([3.0, 2.5, 2.0, 1.5, 1.0, 0.5]))
        X[h] = np.sqrt(S) * Z @ np.diag(sig) @ U.T
        order = np.argsort(-sig)
        want_rows.append(_sign_rule(U[:, order[:r]].T))
        want_lam.append(sig[order] ** 2)
    rows, lam = fit(X, r)
    close(rows, np.stack(want_rows), 1e-10, "closed-form basis rows")
    close(lam, np.stack(want_lam), 1e-10, "closed-form eigenvalues")


def pin_fit_brute_force_plane(L, fit=oracle.fit_basis):
    """d_k = 2: the leading direction maximises the mean squared projection
    (1/S) sum_s (q_s . u)^2 over unit u. Brute force over 400,001 angles."""
    rng = np.random.default_rng(12)
    X = rng.standard_normal((1, 9, 2)) * np.array([1.0, 0.4]) + np.array([0.3, -0.2])
    theta = np.linspace(0.0, np.pi, 400001)
    u = np.stack([np.cos(theta), np.sin(theta)], axis=1)            # [angles][2]
    quot = np.mean((X[0] @ u.T) ** 2, axis=0)
    best = u[int(np.argmax(quot))]
    rows, lam = fit(X, 2)
    assert abs(abs(rows[0, 0] @ best) - 1.0) < 1e-9, "leading direction off the brute-force maximum"
    assert abs(lam[0, 0] - quot.max()) < 1e-9 * quot.max(), "largest eigenvalue is not the maximum"
    assert abs(lam[0, 1] - quot.min()) < 1e-9 * quot.max(), "smallest eigenvalue is not the minimum"


def pin_fit_samples_in_a_subspace(L, fit=oracle.fit_basis):
    """Samples spanning a k-dimensional subspace: the top k rows span exactly it and
    the remaining eigenvalues are zero."""
    rng = np.random.default_rng(13)
    dk, k, S = 7, 3, 20
    P, _ = np.linalg.qr(rng.standard_normal((dk, k)))               # orthonormal columns
    X = (rng.standard_normal((S, k)) @ P.T)[None]
    rows, lam = fit(X, 5)
    proj = rows[0, :k].T @ rows[0, :k]
    close(proj, P @ P.T, 1e-10, "top-k span")
    assert np.all(np.abs(lam[0, k:]) < 1e-12), "eigenvalues beyond the samples' rank"


def pin_fit_invariants(L, fit=oracle.fit_basis):
    """Orthonormal rows; M b_m = lambda_m b_m for M summed sample by sample; the
    eigenvalues decrease and add up to the mean squared norm; the sign rule holds."""
    rng = np.random.default_rng(14)
    X = rng.standard_normal((3, 25, 5)) * np.array([2.0, 1.0, 0.7, 0.5, 0.2])
    rows, lam = fit(X, 3)
    for h in range(3):
        M = np.zeros((5, 5))
        for q in X[h]:
            M += np.outer(q, q)
        M /= X.shape[1]
        close(rows[h] @ rows[h].T, np.eye(3), 1e-12, "orthonormal rows")
        for m in range(3):
            close(M @ rows[h, m], lam[h, m] * rows[h, m], 1e-10, "eigen-equation")
            big = int(np.argmax(np.abs(rows[h, m])))
            assert rows[h, m, big] > 0, "sign rule"
        assert np.all(np.diff(lam[h]) <= 1e-12), "eigenvalues not decreasing"
        close(lam[h].sum(), np.mean(np.sum(X[h] ** 2, axis=1)), 1e-12, "trace")


def pin_fit_is_uncentred(L, fit=oracle.fit_basis):
    """Samples around a large common offset mu: the uncentred second moment is led by
    mu / |mu| (a centred covariance would be led by the spread instead)."""
    rng = np.random.default_rng(15)
    mu = np.array([3.0, -4.0, 0.0, 0.0])
    X = (mu + rng.standard_normal((200, 4)) * np.array([0.0, 0.0, 1.0, 0.1]))[None]
    rows, _ = fit(X, 1)
    assert abs(abs(rows[0, 0] @ mu) / np.linalg.norm(mu) - 1.0) < 1e-3, "not led by the offset"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
FIT_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_fit_")]
