"""TEST INFRASTRUCTURE ONLY: Python access to the fp64 CPU oracle in ``oracle.c``.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. It does not import the HIP library, and the HIP
library does not import it.

The oracle follows the SketchSSM pages (readsearch.ai listing of arXiv
2609.33051, Abstract; agihunt.info summary, "Mechanism details" and "Error
control"): the full state is written once per window, a sketch B S_win is
stored at each window start, and each decode step combines the sketch with
query coefficients c = B q~ plus the exact within-window term. See the header
of ``oracle.c`` for the exact definitions and the readings taken.

Two parts are plain numpy here rather than C: the least-squares read
(``ls_read``) and the offline basis fit (``fit_basis``: top eigenvectors of the
uncentred second moment of sampled queries).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCE = os.path.join(_HERE, "oracle.c")
RULE_IDS = {"mamba2": 0, "gdn": 1, "kda": 2}

_lib = None


def build(out: str = LIB_PATH, extra_flags=(), source: str = SOURCE) -> str:
    """Compile the oracle with gcc (host only, OpenMP, no fast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           *extra_flags, source, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def _load(path: str = LIB_PATH):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_run.restype = ctypes.c_int
    lib.oracle_run.argtypes = [ctypes.c_int] * 7 + [dp] * 15 + [ctypes.c_int] * 2
    lib.oracle_round_bf16.restype = ctypes.c_double
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_rule_step.restype = ctypes.c_int
    lib.oracle_rule_step.argtypes = [ctypes.c_int] * 3 + [dp] * 4 + [ctypes.c_double]
    lib.oracle_transition_matrix.restype = None
    lib.oracle_transition_matrix.argtypes = [ctypes.c_int, ctypes.c_int, dp, dp,
                                             ctypes.c_double, dp]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def lib(path: Optional[str] = None):
    """The loaded oracle library (built on first use if missing)."""
    global _lib
    if path is not None:
        return _load(path)
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
            build()
        _lib = _load(LIB_PATH)
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def transition_matrix(rule: str, k, decay, beta: float = 0.0, _lib_override=None):
    """The token's d_k x d_k transition matrix M_t (dense, fp64)."""
    L = _lib_override or lib()
    k = _f64(k)
    decay = _f64(np.atleast_1d(decay))
    dk = k.shape[0]
    M = np.zeros((dk, dk))
    L.oracle_transition_matrix(RULE_IDS[rule], dk, _ptr(k), _ptr(decay), float(beta), _ptr(M))
    return M


def rule_step(rule: str, S, k, v, decay, beta: float = 0.0, _lib_override=None):
    """One token's state update S <- M_t S + b k v^T; returns the new state."""
    L = _lib_override or lib()
    S = _f64(S).copy()
    k, v = _f64(k), _f64(v)
    decay = _f64(np.atleast_1d(decay))
    dk, dv = S.shape
    rc = L.oracle_rule_step(RULE_IDS[rule], dk, dv, _ptr(S), _ptr(k), _ptr(v), _ptr(decay),
                            float(beta))
    if rc:
        raise RuntimeError("oracle_rule_step failed")
    return S


def run(rule: str, S0, basis, q, k, v, decay, beta, window: int, *,
        want_A: bool = False, want_R: bool = False, want_ls: bool = False,
        sketch_bf16: bool = False, threads: int = 0, _lib_override=None) -> dict:
    """Run T decode steps for U independent units.

    Shapes: S0 [U][dk][dv]; basis [U][r][dk]; q, k [T][U][dk]; v [T][U][dv];
    decay [T][U] or [T][U][dk]; beta [T][U] (None for Mamba-2).
    Returns y_exact, y_replay, y_sketch [T][U][dv]; S_win, Sk [T//W + 1][U][...]
    (window-start states and sketches) and, if asked, A [T][U][dk][dk] and
    R [T][U][dk][dv]. sketch_bf16: the stored sketch is rounded as a bf16 store
    rounds it (to fp32, then to nearest bf16, ties to even) before it is read.
    want_ls: also y_ls [T][U][dv], the sketch read with least-squares coefficients
    (see ls_read) and q~ [T][U][dk].
    """
    L = _lib_override or lib()
    S0, basis, q, k, v, decay = map(_f64, (S0, basis, q, k, v, decay))
    beta = _f64(beta)
    U, dk, dv = S0.shape
    r = basis.shape[1]
    T = q.shape[0]
    nwin = T // window
    out = {
        "y_exact": np.zeros((T, U, dv)),
        "y_replay": np.zeros((T, U, dv)),
        "y_sketch": np.zeros((T, U, dv)),
        "S_win": np.zeros((nwin + 1, U, dk, dv)),
        "Sk": np.zeros((nwin + 1, U, r, dv)),
        "A": np.zeros((T, U, dk, dk)) if want_A else None,
        "R": np.zeros((T, U, dk, dv)) if want_R else None,
        "qt": np.zeros((T, U, dk)) if want_ls else None,
    }
    rc = L.oracle_run(RULE_IDS[rule], U, dk, dv, r, window, T,
                      _ptr(S0), _ptr(basis), _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta),
                      _ptr(out["y_exact"]), _ptr(out["y_replay"]), _ptr(out["y_sketch"]),
                      _ptr(out["S_win"]), _ptr(out["Sk"]), _ptr(out["A"]), _ptr(out["R"]),
                      _ptr(out["qt"]), int(bool(sketch_bf16)), int(threads))
    if rc:
        raise RuntimeError("oracle_run failed")
    if want_ls:
        out["y_ls"] = ls_read(out, window)
    return out


# Rank decisions of the least-squares read: a singular value of the sketch counts
# as zero below this fraction of the largest one.
LS_RCOND = 1e-5


def ls_read(out: dict, window: int) -> np.ndarray:
    """The sketch read with least-squares coefficients (a reading of the pages'
    "state-weighted query approximation", readsearch.ai listing of arXiv 2609.33051,
    Abstract): at step t of a window, c minimises || S_win^T q~ - Sk^T c || (the
    smallest such c when Sk is rank-deficient) and y = Sk^T c + R^T q, where
    R^T q = y_replay - S_win^T q~. Sk^T c is the orthogonal projection of the exact
    window-start read S_win^T q~ onto the span of the sketch rows.
    """
    T, U, dv = out["y_replay"].shape
    y = np.empty((T, U, dv))
    for t in range(T):
        win = t // window
        for u in range(U):
            Sw, Sk, qt = out["S_win"][win, u], out["Sk"][win, u], out["qt"][t, u]
            exact = Sw.T @ qt                                  # S_win^T q~, [dv]
            c = np.linalg.lstsq(Sk.T, exact, rcond=LS_RCOND)[0]
            y[t, u] = Sk.T @ c + (out["y_replay"][t, u] - exact)
    return y


def fit_basis(samples, rank: int):
    """The offline basis fit of the C2 workload, as a plain definition (the pages fix the
    basis vectors offline, readsearch.ai listing of arXiv 2609.33051, Abstract; the
    query-basis idea, agihunt.info summary, "Mechanism details"; the recipe, top-r PCA
    directions of sampled queries made orthonormal, is read from the workload's
    description). Per head h, with X = samples[h] ([S][d_k]):

      M = X^T X / S   (the uncentred second moment of the samples),
      rows m = 0 .. rank-1: unit eigenvectors of M for its rank largest eigenvalues,
      in decreasing order of eigenvalue, each signed so that its entry of largest
      magnitude (the first such entry on a tie) is positive.

    Returns (basis [H][rank][d_k], eigenvalues [H][d_k] in decreasing order), fp64.
    The rows are unique (up to the sign rule) only where the eigenvalue gaps around
    them are non-zero; callers compare subspaces where they are not.
    """
    X = _f64(samples)
    H, S, dk = X.shape
    out = np.empty((H, rank, dk))
    lam = np.empty((H, dk))
    for h in range(H):
        M = X[h].T @ X[h] / S
        w, V = np.linalg.eigh(M)                 # ascending eigenvalues, orthonormal columns
        order = np.argsort(-w, kind="stable")
        lam[h] = w[order]
        for m in range(rank):
            v = V[:, order[m]]
            big = int(np.argmax(np.abs(v)))
            out[h, m] = v if v[big] > 0 else -v
    return out, lam


def round_bf16(x: float, _lib_override=None) -> float:
    """x rounded as a bf16 store rounds it (to fp32, then to nearest bf16, ties to even)."""
    return float((_lib_override or lib()).oracle_round_bf16(float(x)))


def max_threads() -> int:
    return int(lib().oracle_max_threads())
