"""Shared machinery of the GPU parity tests: seeded inputs on the device, the
decode run through the library, the oracle on sampled units, and the
comparison at the stated tolerances.

Tolerances (fp32 state, bf16 inputs): outputs within 1e-3 relative per
(unit, step) for both reads, state and sketch within 1e-4 relative per unit
after every window. The error of an output vector is ||got - ref|| / max(||ref||,
1e-6 * rms_rows ||ref||); the state's is the Frobenius ratio per unit.

State and sketch are also compared element by element: every element's error,
over the largest magnitude of its unit's state (or sketch), must be within the
same 1e-4.

A bf16 sketch is compared element by element with the oracle's sketch rounded
the same way (fp32, then nearest bf16, ties to even), using oracle values only.
The kernel's fp32 sketch value before rounding may differ from the oracle's
unrounded value x by the fp32 tolerance t = 1e-4 of the unit's sketch scale, and
rounding is monotone, so the stored element must lie in
[bf16(x - t), bf16(x + t)]: exactly bf16(x) wherever that interval is a single
value (x is not within t of a rounding midpoint), and at most 1% of elements may
differ at all. Through y = Sk^T c + intra, those allowed differences move y_j by
at most sum_m |c_m| (bf16(x_mj + t) - bf16(x_mj - t)), with c = B q~ from the
oracle; the sketch read must meet the fp32 tolerance beyond that.
"""
from __future__ import annotations

import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import workloads
import sketched_recurrent_state_amd as ssm
from sketched_recurrent_state_amd.decoder import WindowedDecoder

Y_TOL = 1e-3
S_TOL = 1e-4


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dims_of(cfg: workloads.Config, sketch_dtype: str = "f32") -> ssm.Dims:
    return ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k, cfg.d_v,
                         cfg.window, cfg.rank, sketch_dtype)


def _to_dev(x: np.ndarray, dev) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


class Inputs:
    """Every step's inputs on the device ([T][N][H]...) plus host copies of a unit sample."""

    def __init__(self, cfg: workloads.Config, units: np.ndarray, steps: int, dev="cuda",
                 threads: int = 8):
        self.cfg, self.units, self.steps = cfg, np.asarray(units), steps
        U = cfg.units
        t0 = time.time()
        with ThreadPoolExecutor(threads) as ex:
            s0 = list(ex.map(lambda n: workloads.initial_state(cfg, [n]), range(cfg.batch)))
        S0 = np.concatenate(s0)
        self.S0 = _to_dev(S0, dev)
        self.host_S0 = S0.reshape(U, cfg.d_k, cfg.d_v)[self.units].astype(np.float64)
        del S0, s0
        B = workloads.basis(cfg)
        self.basis = _to_dev(B, dev)
        self.host_basis = B[self.units % cfg.heads].astype(np.float64)
        self.q, self.k, self.v, self.decay, self.beta = [], [], [], [], []
        hq, hk, hv, hd, hb = [], [], [], [], []
        with ThreadPoolExecutor(threads) as ex:
            for t, si in enumerate(ex.map(lambda t: workloads.step_inputs(cfg, t), range(steps))):
                self.q.append(_to_dev(si.q, dev))
                self.k.append(_to_dev(si.k, dev))
                self.v.append(_to_dev(si.v, dev))
                self.decay.append(_to_dev(si.decay, dev))
                self.beta.append(_to_dev(si.beta, dev) if si.beta is not None else None)
                flat = lambda x, e: x.reshape((U,) + ((e,) if e else ()))[self.units]
                hq.append(workloads.widen(flat(si.q, cfg.d_k)))
                hk.append(workloads.widen(flat(si.k, cfg.d_k)))
                hv.append(workloads.widen(flat(si.v, cfg.d_v)))
                hd.append(flat(si.decay, cfg.d_k if cfg.per_channel_decay else 0).astype(np.float64))
                hb.append(flat(si.beta, 0).astype(np.float64) if si.beta is not None else None)
        self.host = dict(q=np.stack(hq), k=np.stack(hk), v=np.stack(hv), decay=np.stack(hd),
                         beta=np.stack(hb) if hb[0] is not None else None)
        note(f"inputs {cfg.name}: {steps} steps, {U} units, {time.time() - t0:.1f}s")


def run_gpu(cfg: workloads.Config, inp: Inputs, *, fused: bool = True, check_state_frozen=True,
            sketch_dtype: str = "f32", coefficients: str = "projection"):
    """Decode all steps with both reads; returns sampled outputs and window snapshots."""
    d = dims_of(cfg, sketch_dtype)
    U, W = cfg.units, cfg.window
    idx = torch.as_tensor(inp.units, device=inp.S0.device)
    state = inp.S0.clone()
    dec = WindowedDecoder(d, state, inp.basis, read="both", fused=fused,
                          coefficients=coefficients)
    dec.refresh()
    ys, yf = [], []
    S_snap = [state.view(U, -1)[idx].cpu().numpy()]
    Sk_snap = [dec.sketch.view(U, -1)[idx].float().cpu().numpy()]
    frozen_state = state.clone() if check_state_frozen else None
    frozen_sketch = dec.sketch.clone() if check_state_frozen else None
    y = torch.empty((cfg.batch, cfg.heads, cfg.d_v), device=state.device)
    y2 = torch.empty_like(y)
    for t in range(inp.steps):
        tau = t % W + 1
        if tau == W and check_state_frozen:
            # decode steps never write the state or the sketch
            assert torch.equal(state, frozen_state), f"state written inside window at step {t}"
            assert torch.equal(dec.sketch, frozen_sketch), f"sketch written inside window at {t}"
        dec.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t], y=y, y_full=y2)
        ys.append(y.view(U, -1)[idx].cpu().numpy())
        yf.append(y2.view(U, -1)[idx].cpu().numpy())
        if tau == W:
            S_snap.append(state.view(U, -1)[idx].cpu().numpy())
            Sk_snap.append(dec.sketch.view(U, -1)[idx].float().cpu().numpy())
            if check_state_frozen:
                frozen_state.copy_(state)
                frozen_sketch.copy_(dec.sketch)
    torch.cuda.synchronize()
    n = len(inp.units)
    return dict(y_sketch=np.stack(ys).astype(np.float64), y_full=np.stack(yf).astype(np.float64),
                S=np.stack(S_snap).reshape(-1, n, cfg.d_k, cfg.d_v).astype(np.float64),
                Sk=np.stack(Sk_snap).reshape(-1, n, cfg.rank, cfg.d_v).astype(np.float64),
                final_state=state, sketch=dec.sketch, read_map=dec.read_map)


def run_gpu_full(cfg: workloads.Config, inp: Inputs, *, fused: bool = True, keep_buffers=False):
    """The exact buffered path alone (read="full"): every step appends the current token
    (inside the full-read kernel when fused, else by a separate append launch) and reads
    y = S_win^T q~ + R^T q from the full state; one update per window. Returns sampled
    outputs, window-start states and, with keep_buffers, the window buffer after every step."""
    d = dims_of(cfg)
    U, W = cfg.units, cfg.window
    idx = torch.as_tensor(inp.units, device=inp.S0.device)
    state = inp.S0.clone()
    dec = WindowedDecoder(d, state, None, read="full", fused=fused)
    y = torch.empty((cfg.batch, cfg.heads, cfg.d_v), device=state.device)
    ys, S_snap, bufs = [], [state.view(U, -1)[idx].cpu().numpy()], []
    for t in range(inp.steps):
        dec.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t], y_full=y)
        ys.append(y.view(U, -1)[idx].cpu().numpy())
        if keep_buffers:
            bufs.append(tuple(None if b is None else b.clone()
                              for b in (dec.k_buf, dec.v_buf, dec.decay_buf, dec.beta_buf)))
        if (t + 1) % W == 0:
            S_snap.append(state.view(U, -1)[idx].cpu().numpy())
    torch.cuda.synchronize()
    n = len(inp.units)
    return dict(y=np.stack(ys).astype(np.float64),
                S=np.stack(S_snap).reshape(-1, n, cfg.d_k, cfg.d_v).astype(np.float64),
                bufs=bufs)


def run_oracle(cfg: workloads.Config, inp: Inputs, threads: int = 0, sketch_bf16: bool = False,
               want_ls: bool = False):
    h = inp.host
    return oracle.run(cfg.rule, inp.host_S0, inp.host_basis, h["q"], h["k"], h["v"], h["decay"],
                      h["beta"], cfg.window, threads=threads, sketch_bf16=sketch_bf16,
                      want_ls=want_ls)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """One bf16 unit in the last place at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), np.finfo(np.float32).tiny)))
    return np.exp2(e - 7)


def rel_diff_rows(diff: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-vector norm of diff over the last axis, relative to ref's."""
    num = np.linalg.norm(diff, axis=-1)
    nref = np.linalg.norm(ref, axis=-1)
    floor = 1e-6 * np.sqrt(np.mean(nref ** 2)) if nref.size else 0.0
    return num / np.maximum(nref, floor)


def rel_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-vector relative error over the last axis."""
    return rel_diff_rows(got - ref, ref)


def rel_mats(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    a = got.reshape(got.shape[:2] + (-1,))
    b = ref.reshape(ref.shape[:2] + (-1,))
    return rel_rows(a, b)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """x rounded as a bf16 store rounds it: to fp32, then to nearest bf16, ties to even."""
    return workloads.widen(workloads.to_bf16_bits(np.asarray(x, dtype=np.float32)))


def bf16_window(sk_exact: np.ndarray, s_tol: float):
    """The stored bf16 values the kernel may hold for each sketch element: [lo, hi] =
    [bf16(x - t), bf16(x + t)] with x the oracle's unrounded sketch and t the fp32
    tolerance, s_tol times the unit's largest sketch magnitude. Oracle values only."""
    scale = np.max(np.abs(sk_exact).reshape(sk_exact.shape[:2] + (-1,)), axis=-1)
    t = s_tol * scale[:, :, None, None]
    return bf16_round(sk_exact - t), bf16_round(sk_exact + t)


def bf16_read_slack(cfg, ref, ref_exact, host_basis, s_tol=None) -> np.ndarray:
    """What a bf16 sketch's own rounding may add to the sketch read, [T][U][dv], from oracle
    values only: sum_m |c_m| (hi_mj - lo_mj), with c = B q~ (the oracle's q~; run_oracle(...,
    want_ls=True) returns it) and [lo, hi] the window of bf16_window around the oracle's
    unrounded sketch (ref_exact, a run without sketch rounding). Zero for every element that
    is not within the fp32 tolerance of a bf16 rounding midpoint."""
    s_tol = S_TOL if s_tol is None else s_tol
    c = np.einsum("urk,tuk->tur", host_basis, ref["qt"])              # [T][U][r]
    win = np.arange(c.shape[0]) // cfg.window
    lo, hi = bf16_window(ref_exact["Sk"][:win[-1] + 1], s_tol)
    return np.einsum("tur,turj->tuj", np.abs(c), (hi - lo)[win])


def element_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Largest element error over the largest magnitude of its unit, for [W][U][...] stacks
    of per-unit matrices."""
    d = np.abs(got - ref).reshape(got.shape[:2] + (-1,))
    s = np.abs(ref).reshape(ref.shape[:2] + (-1,))
    return float((np.max(d, axis=-1) / np.maximum(np.max(s, axis=-1), 1e-30)).max())


def assert_mats(got: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    """Per-unit Frobenius ratio and per-element error (over the unit's largest magnitude) of
    [W][U][...] stacks, both within tol; returns the larger."""
    e_f = float(rel_mats(got, ref).max())
    e_e = element_err(got, ref)
    assert e_f <= tol, f"{what}: max Frobenius rel err {e_f:.3e} > {tol}"
    assert e_e <= tol, f"{what}: max element err {e_e:.3e} (of the unit's largest) > {tol}"
    return max(e_f, e_e)


def compare(cfg, got, ref, *, y_tol=Y_TOL, s_tol=S_TOL, sketch_bf16: bool = False,
            host_basis=None, ref_exact=None) -> dict:
    """Assert parity; returns the error summary. With sketch_bf16, ref is an oracle run with
    the sketch rounded (want_ls=True, for q~), ref_exact one without (its unrounded sketch),
    and host_basis the oracle run's basis rows per unit: together they set the stored
    sketch's allowed values and the read's rounding slack (bf16_read_slack)."""
    slack = bf16_read_slack(cfg, ref, ref_exact, host_basis, s_tol) if sketch_bf16 else 0.0
    d_sk = np.maximum(np.abs(got["y_sketch"] - ref["y_sketch"]) - slack, 0.0)
    e_sk = rel_diff_rows(d_sk, ref["y_sketch"])
    e_ex = rel_rows(got["y_full"], ref["y_exact"])
    # element by element, on the row's scale
    scale = np.maximum(np.max(np.abs(ref["y_exact"]), axis=-1, keepdims=True), 1e-30)
    el_ex = np.max(np.abs(got["y_full"] - ref["y_exact"]) / scale)
    scale_s = np.maximum(np.max(np.abs(ref["y_sketch"]), axis=-1, keepdims=True), 1e-30)
    el_sk = np.max(d_sk / scale_s)
    nw = got["S"].shape[0]
    e_S = rel_mats(got["S"], ref["S_win"][:nw])
    el_S = element_err(got["S"], ref["S_win"][:nw])
    e_Sk = rel_mats(got["Sk"], ref["Sk"][:nw])
    el_Sk = element_err(got["Sk"], ref["Sk"][:nw])
    if sketch_bf16:
        lo, hi = bf16_window(ref_exact["Sk"][:nw], s_tol)
        outside = (got["Sk"] < lo) | (got["Sk"] > hi)
        frac_diff = float(np.mean(got["Sk"] != ref["Sk"][:nw]))
        frac_window = float(np.mean(hi > lo))
    approx = rel_rows(ref["y_sketch"], ref["y_exact"])
    summary = dict(config=cfg.name, y_sketch_max=float(e_sk.max()), y_exact_max=float(e_ex.max()),
                   y_sketch_elem_max=float(el_sk), y_exact_elem_max=float(el_ex),
                   S_max=float(e_S.max()), S_elem_max=el_S, Sk_max=float(e_Sk.max()),
                   Sk_elem_max=el_Sk, approx_err_mean=float(approx.mean()),
                   approx_err_max=float(approx.max()))
    note(f"parity {summary}")
    assert e_sk.max() <= y_tol, f"sketch read: max rel err {e_sk.max():.3e} > {y_tol}"
    assert e_ex.max() <= y_tol, f"exact read: max rel err {e_ex.max():.3e} > {y_tol}"
    assert el_sk <= y_tol and el_ex <= y_tol, f"element error {el_sk:.3e}/{el_ex:.3e}"
    assert e_S.max() <= s_tol, f"state: max rel err {e_S.max():.3e} > {s_tol}"
    assert el_S <= s_tol, f"state: max element err {el_S:.3e} (of the unit's largest) > {s_tol}"
    if sketch_bf16:
        note(f"bf16 sketch: {frac_diff:.2e} of elements differ from the oracle's rounding, "
             f"{frac_window:.2e} may; {int(outside.sum())} outside their window")
        assert not outside.any(), f"bf16 sketch: {int(outside.sum())} elements outside [lo, hi]"
        assert frac_diff <= 0.01, f"bf16 sketch: {frac_diff:.3f} of elements differ"
    else:
        assert e_Sk.max() <= s_tol, f"sketch: max rel err {e_Sk.max():.3e} > {s_tol}"
        assert el_Sk <= s_tol, f"sketch: max element err {el_Sk:.3e} (of the unit's largest) > {s_tol}"
    return summary


def run_gpu_recurrent(cfg: workloads.Config, inp: Inputs):
    """The per-token recurrent decode: sampled outputs and states after every token."""
    from sketched_recurrent_state_amd.decoder import RecurrentDecoder
    d = dims_of(cfg)
    U = cfg.units
    idx = torch.as_tensor(inp.units, device=inp.S0.device)
    state = inp.S0.clone()
    dec = RecurrentDecoder(d, state)
    y = torch.empty((cfg.batch, cfg.heads, cfg.d_v), device=state.device)
    ys, Ss = [], [state.view(U, -1)[idx].cpu().numpy()]
    for t in range(inp.steps):
        dec.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t], y=y)
        ys.append(y.view(U, -1)[idx].cpu().numpy())
        Ss.append(state.view(U, -1)[idx].cpu().numpy())
    torch.cuda.synchronize()
    n = len(inp.units)
    return dict(y=np.stack(ys).astype(np.float64),
                S=np.stack(Ss).reshape(-1, n, cfg.d_k, cfg.d_v).astype(np.float64))


def compare_recurrent(cfg, got, inp, *, y_tol=Y_TOL, s_tol=S_TOL) -> dict:
    """Per-token path vs the oracle's exact read and its state after every token (W = 1)."""
    ref = run_oracle(cfg.with_(window=1), inp)
    e_y = rel_rows(got["y"], ref["y_exact"])
    summary = dict(config=cfg.name, y_max=float(e_y.max()))
    assert e_y.max() <= y_tol, f"recurrent read: max rel err {e_y.max():.3e}"
    summary["S_max"] = assert_mats(got["S"], ref["S_win"], s_tol, "recurrent state")
    note(f"recurrent parity {summary}")
    return summary
