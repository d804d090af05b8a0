"""GPU parity of the offline basis fit (ssm_fit_basis) against the oracle's fp64 fit.

The rows are eigenvectors, so they are determined only as far as the eigenvalues
around them are separated. The comparison therefore goes through subspaces, with
tolerances from the arithmetic:
  * the kernel forms M = X^T X / S in fp32 from inputs exact in fp32: every entry is
    a sum of S products, off by at most S * 2^-24 * sqrt(M_ii M_jj) in magnitude;
    fp32 Jacobi adds a backward error of a few d_k * 2^-24 * |M|. With
    E = (S + 8 d_k) * 2^-24 * lambda_max as the allowance for |dM|,
  * the span of the top k rows moves by at most E / gap_k (Davis-Kahan), where
    gap_k = lambda_k - lambda_(k+1) (zero-based: lambda[k-1] - lambda[k]); it is
    compared whenever gap_k > 10 E, at 2 E / gap_k + 1e-6 in the spectral norm;
  * a row whose eigenvalue is separated from both neighbours by more than 10 E is
    compared itself, at 4 E / gap + 1e-5, after the sign rule (when the rule's
    largest entry is unambiguous on both sides);
  * each row's Rayleigh quotient b^T M b matches its eigenvalue within 4 E + 1e-7 lambda_max;
  * rows are orthonormal within 1e-5 and signed by the rule where unambiguous.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import sketched_recurrent_state_amd as ssm
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def planted(heads, S, dk, r, in_dtype, seed):
    """Samples with a chosen spectrum: the top r eigenvalues spread evenly over
    [0.5, 1] (gaps 1 / (2r)), the others below 0.3 (zero past the S-th when S < d_k),
    times a per-head scale."""
    rng = np.random.default_rng([0xF17, seed, dk, r, S])
    X = np.empty((heads, S, dk), np.float32)
    n = min(S, dk)
    for h in range(heads):
        U, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        lam = np.concatenate([1.0 - 0.5 * np.arange(r) / r, 0.3 * (1.0 - np.arange(dk - r) / dk)])
        sig = np.sqrt(lam[:n]) * rng.uniform(0.5, 2.0)
        Z, _ = np.linalg.qr(rng.standard_normal((S, n)))
        X[h] = np.sqrt(S) * Z @ np.diag(sig) @ U[:, :n].T
    return pack(X, in_dtype)


def gaussian(heads, S, dk, in_dtype, seed):
    rng = np.random.default_rng([0x6A55, seed, dk, S])
    X = rng.standard_normal((heads, S, dk)).astype(np.float32) * np.linspace(2.0, 0.2, dk, dtype=np.float32)
    return pack(X, in_dtype)


def pack(X, in_dtype):
    return workloads.to_bf16_bits(X) if in_dtype == "bf16" else X.astype(np.float32)


def fit_gpu(samples, r, in_dtype):
    heads, S, dk = samples.shape
    d = ssm.Dims.make("mamba2", in_dtype, 1, heads, dk, 32, 1, r)
    x = H._to_dev(samples, "cuda")
    out = torch.full((heads, r, dk), float("nan"), device="cuda")
    H.note(f"fit_basis H={heads} S={S} d_k={dk} r={r} {in_dtype}")
    ssm.fit_basis(d, x, S, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def sign_unambiguous(row, margin=1e-5):
    a = np.sort(np.abs(row))[::-1]
    return len(a) < 2 or a[0] - a[1] > margin


def check_fit(samples, got, r, what):
    X = workloads.widen(samples)                      # exact inputs, fp64
    rows_o, lam_o = oracle.fit_basis(X, r)
    heads, S, dk = X.shape
    u = 2.0 ** -24
    assert np.all(np.isfinite(got)), f"{what}: non-finite basis"
    for h in range(heads):
        M = X[h].T @ X[h] / S
        lam = lam_o[h]
        lmax = max(float(lam[0]), 1e-30)
        E = (S + 8 * dk) * u * lmax
        B = got[h].astype(np.float64)
        err = np.abs(B @ B.T - np.eye(r)).max()
        assert err <= 1e-5, f"{what} h={h}: rows not orthonormal ({err:.2e})"
        for m in range(r):
            quot = B[m] @ M @ B[m]
            assert abs(quot - lam[m]) <= 4 * E + 1e-7 * lmax, \
                f"{what} h={h} row {m}: Rayleigh quotient {quot:.6e} vs eigenvalue {lam[m]:.6e}"
            if sign_unambiguous(B[m]):
                assert B[m][int(np.argmax(np.abs(B[m])))] > 0, f"{what} h={h} row {m}: sign rule"
        compared = 0
        for k in range(1, r + 1):
            if k == dk:
                continue
            gap = lam[k - 1] - lam[k]
            if gap > 10 * E:
                Pg, Po = B[:k].T @ B[:k], rows_o[h, :k].T @ rows_o[h, :k]
                e = np.linalg.norm(Pg - Po, 2)
                assert e <= 2 * E / gap + 1e-6, \
                    f"{what} h={h}: span of the top {k} rows off by {e:.2e} (gap {gap:.2e}, E {E:.2e})"
                compared += 1
        for m in range(r):
            lo = lam[m - 1] - lam[m] if m > 0 else np.inf
            hi = lam[m] - lam[m + 1] if m + 1 < dk else np.inf
            g = min(lo, hi)
            if g > 10 * E and sign_unambiguous(B[m]) and sign_unambiguous(rows_o[h, m]):
                e = np.linalg.norm(B[m] - rows_o[h, m])
                assert e <= 4 * E / g + 1e-5, f"{what} h={h} row {m}: off by {e:.2e} (gap {g:.2e})"
    return compared


PLANTED = [  # (d_k, r, S, input type, heads)
    (16, 4, 50, "f32", 3),
    (16, 15, 16, "bf16", 2),
    (32, 8, 64, "bf16", 3),
    (64, 16, 100, "f32", 2),
    (64, 3, 33, "bf16", 2),      # a ragged last staging block
    (128, 8, 4096, "bf16", 2),   # the workload's sample count
    (128, 32, 1000, "f32", 2),   # the largest rank
]


@pytest.mark.parametrize("dk,r,S,in_dtype,heads", PLANTED,
                         ids=[f"dk{c[0]}_r{c[1]}_S{c[2]}_{c[3]}" for c in PLANTED])
def test_planted_spectrum(dk, r, S, in_dtype, heads):
    x = planted(heads, S, dk, r, in_dtype, seed=1)
    got = fit_gpu(x, r, in_dtype)
    n = check_fit(x, got, r, f"planted dk={dk} r={r} S={S}")
    assert n > 0, "no subspace was separated enough to compare"


GAUSSIAN = [  # few samples: the spectrum comes from the data; rank-deficient cases
    (128, 5, 7, "bf16", 2),
    (32, 8, 3, "f32", 2),        # fewer samples than rows: rows past the third span the null space
    (128, 1, 1, "bf16", 3),      # one sample: the row is that sample, normalised
    (64, 12, 500, "f32", 2),
]


@pytest.mark.parametrize("dk,r,S,in_dtype,heads", GAUSSIAN,
                         ids=[f"dk{c[0]}_r{c[1]}_S{c[2]}_{c[3]}" for c in GAUSSIAN])
def test_sampled_spectrum(dk, r, S, in_dtype, heads):
    x = gaussian(heads, S, dk, in_dtype, seed=2)
    got = fit_gpu(x, r, in_dtype)
    check_fit(x, got, r, f"gaussian dk={dk} r={r} S={S}")
    if S == 1:
        q = workloads.widen(x)[:, 0]
        want = q / np.linalg.norm(q, axis=1, keepdims=True)
        want *= np.sign(want[np.arange(len(q)), np.argmax(np.abs(want), axis=1)])[:, None]
        np.testing.assert_allclose(got[:, 0], want, atol=2e-6)


def test_workload_recipe():
    """The Mamba-2 workload's recipe: 4096 queries per head drawn like its decode queries."""
    cfg = workloads.C2.with_(heads=4)
    x = workloads.pca_samples(cfg)
    got = fit_gpu(x, cfg.rank, cfg.in_dtype)
    assert check_fit(x, got, cfg.rank, "workload recipe") > 0


def test_zero_samples():
    """M = 0: every direction is an eigenvector; the rows are still orthonormal and finite."""
    x = np.zeros((2, 40, 64), np.float32)
    got = fit_gpu(x, 6, "f32")
    check_fit(x, got, 6, "zero samples")


def test_fit_feeds_the_decode():
    """The fitted basis in the decode path: the GPU decodes with the GPU's fit and the
    oracle with its own fit of the same samples. The planted spectrum separates the top
    eight eigenvalues by 1/16, so the two bases differ by ~E / gap ~ 1e-6 and the
    outputs, states and sketches must agree at the decode tolerances."""
    cfg = workloads.C2.with_(batch=2, heads=4, steps=10)
    x = planted(cfg.heads, 512, cfg.d_k, cfg.rank, cfg.in_dtype, seed=3)
    basis_gpu = fit_gpu(x, cfg.rank, cfg.in_dtype)
    basis_oracle, _ = oracle.fit_basis(workloads.widen(x), cfg.rank)
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    inp.basis = torch.from_numpy(np.ascontiguousarray(basis_gpu)).cuda()
    inp.host_basis = basis_oracle[inp.units % cfg.heads]
    got = H.run_gpu(cfg, inp)
    ref = H.run_oracle(cfg, inp)
    H.compare(cfg, got, ref)


def test_fitted_basis_makes_low_rank_queries_exact():
    """The method's premise end to end: when the queries lie in an r-dimensional subspace per
    head, a basis fitted on the device from sampled queries spans it, and for Mamba-2 (whose
    transposed transitions only scale q, so q~ stays in that subspace) the sketch read equals
    the exact read. fp32 inputs keep the queries in the subspace up to fp32 rounding (~6e-8
    relative); the fitted span is off by ~E / gap with E ~ (S + 8 d_k) 2^-24, so the sketch
    read must agree with the exact read to ~1e-5. The oracle decodes with its own fp64 fit of
    the same samples."""
    cfg = workloads.C2.with_(batch=4, heads=4, steps=16, in_dtype="f32")
    H_, dk, r = cfg.heads, cfg.d_k, cfg.rank
    rng = np.random.default_rng([0x10F1, dk, r])
    U = np.stack([np.linalg.qr(rng.standard_normal((dk, r)))[0] for _ in range(H_)])  # [H][dk][r]
    draw = lambda lead: (np.einsum("hkr,...hr->...hk", U, rng.standard_normal(lead + (H_, r)))
                         / np.sqrt(r)).astype(np.float32)
    samples = np.ascontiguousarray(np.moveaxis(draw((512,)), 0, 1))  # [H][S][dk]
    basis_gpu = fit_gpu(samples, r, "f32")
    basis_oracle, lam = oracle.fit_basis(workloads.widen(samples), r)
    assert np.all(lam[:, r - 1] > 1e3 * np.abs(lam[:, r:]).max(initial=0.0) + 1e-3), \
        "the samples do not span r directions"
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    hq = []
    for t in range(cfg.steps):
        q = draw((cfg.batch,))                                      # [N][H][dk]
        inp.q[t] = torch.from_numpy(q).cuda()
        hq.append(q.reshape(cfg.units, dk)[inp.units].astype(np.float64))
    inp.host["q"] = np.stack(hq)
    inp.basis = torch.from_numpy(np.ascontiguousarray(basis_gpu)).cuda()
    inp.host_basis = basis_oracle[inp.units % H_]
    got = H.run_gpu(cfg, inp)
    ref = H.run_oracle(cfg, inp)
    H.compare(cfg, got, ref)
    e_oracle = H.rel_rows(ref["y_sketch"], ref["y_exact"]).max()
    e_gpu = H.rel_rows(got["y_sketch"], got["y_full"]).max()
    H.note(f"sketch vs exact read, low-rank queries: oracle {e_oracle:.2e}, GPU {e_gpu:.2e}")
    assert e_oracle <= 1e-5, f"oracle: sketch read off the exact read by {e_oracle:.2e}"
    assert e_gpu <= 1e-4, f"GPU: sketch read off the exact read by {e_gpu:.2e}"
