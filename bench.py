#!/usr/bin/env python3
"""Decode-throughput benchmark of the SketchSSM windowed decode path on one GPU.

Workload (default): a Gated DeltaNet decode layer, N=256 sequences x H=32
heads, 128 x 128 fp32 state per (sequence, head), bf16 q/k/v, window W=8,
sketch rank r=8. One timed step is one decode step of the whole layer: the
current token is appended to the window buffer and the output is read from
the sketch (one fused launch); after every W-th step the fused update +
refresh writes the state once and stores the new sketch. The timed steps are
whole windows, so every window's state write is inside the timed region:
--steps and --warmup are rounded up to multiples of W, and the JSON line
reports both the requested and the timed (effective) counts. The timed steps
are captured once into a HIP graph and the headline times one replay of it,
bracketed by device synchronisations; the same steps launched one by one are
timed too (eager: enqueued right behind the warmup steps, with HIP events
around every update + refresh launch for the roofline).

Prints one JSON line. Extra fields: per-kernel times, two comparison paths on
the same tokens (the exact buffered full read, and the per-token recurrent
decode that updates and reads the whole state every step), the byte model,
the sketch's approximation error over the workload's T decode steps (both
coefficient kinds), and the oracle's CPU rate on a bounded sample.

    python bench.py [--steps 64] [--warmup 16] [--config c3]
    python bench.py --sweep c5     # the 12 (r, W) points of the GDN sweep, one line each
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the update + refresh kernel on this workload
TRAFFIC_FILE = os.path.join(HERE, "profiles", "update_refresh_gdn_n256_h32_128x128_w8_r8.pmc.md")
KERNEL_SOURCES = ["common.hpp", "update_body.hpp", "update_refresh.hpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, "sketched_recurrent_state_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def plan_steps(steps: int, warmup: int, window: int) -> tuple:
    """Timed and warmup step counts rounded up to whole windows (at least one timed window),
    so that every window's update + refresh falls inside the region it belongs to."""
    up = lambda x: -(-max(int(x), 0) // window) * window
    return max(up(steps), window), up(warmup)


def bytes_model(cfg, sk_bytes: int = 4, ls: bool = False) -> dict:
    """Algorithmic HBM bytes per unit (sequence, head); sk_bytes per sketch element;
    ls: least-squares coefficients (the per-unit read map [r][d_k] fp32 is written by
    the update and read every step)."""
    s_in = 2 if cfg.in_dtype == "bf16" else 4
    g = {"mamba2": 4, "gdn": 8, "kda": 4 * cfg.d_k + 4}[cfg.rule]
    tok = (cfg.d_k + cfg.d_v) * s_in + g
    W, r, dk, dv = cfg.window, cfg.rank, cfg.d_k, cfg.d_v
    tau_mean = (W + 1) / 2
    # per decode step: q + the current token (appended: read once, written once)
    #   + the older buffered tokens + y; plus the sketch or the full state
    step_common = dk * s_in + tok + (tau_mean - 1) * tok + tok + 4 * dv
    rmap = 4 * r * dk if ls else 0
    sketch_step = sk_bytes * r * dv + rmap + step_common
    full_step = 4 * dk * dv + step_common
    update = 8 * dk * dv + sk_bytes * r * dv + rmap + W * tok  # S in and out, Sk (+map), buffer
    update_no_refresh = 8 * dk * dv + W * tok
    return dict(tok=tok, sketch_step=sketch_step, full_step=full_step, update=update,
                update_no_refresh=update_no_refresh,
                state_bytes_sketch=sk_bytes * r * dv, state_bytes_full=4 * dk * dv,
                amortized_sketch=sketch_step + update / W,
                amortized_full=full_step + update_no_refresh / W)


def metric_name(cfg) -> str:
    if cfg.name == "c3":
        return "decode steps/sec and achieved HBM GB/s (% roofline), GDN 128×128 state, B=256, r=8"
    rule = {"mamba2": "Mamba-2", "gdn": "GDN", "kda": "KDA"}[cfg.rule]
    return (f"decode steps/sec and achieved HBM GB/s (% roofline), {rule} {cfg.d_k}×{cfg.d_v} "
            f"state, B={cfg.batch}, H={cfg.heads}, W={cfg.window}, r={cfg.rank}")


def cpu_model() -> str:
    """The host CPU's model name (Linux), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def error_summary(num_sq, den_sq) -> dict:
    """Relative error of the sketch read against the exact read from per-(unit, step) squared
    norms: the global Frobenius ratio over every output of the run, and the distribution of
    the per-vector ratios ||y_sketch - y_exact|| / ||y_exact||."""
    num_sq = np.asarray(num_sq, dtype=np.float64).ravel()
    den_sq = np.asarray(den_sq, dtype=np.float64).ravel()
    e = np.sqrt(num_sq) / np.maximum(np.sqrt(den_sq), 1e-30)
    return {"frobenius": float(np.sqrt(num_sq.sum() / max(den_sq.sum(), 1e-300))),
            "mean": float(e.mean()), "p50": float(np.median(e)),
            "p99": float(np.quantile(e, 0.99)), "max": float(e.max()), "vectors": int(e.size)}


class Layer:
    """One workload's inputs resident on the device, and the timed legs run over them.

    `steps_host` / `inputs` hold every step's tokens (host arrays / device tensors); the
    library is called with raw device addresses, so the timed loops pay no marshalling."""

    def __init__(self, cfg, n_steps: int, dev, torch, ssm, workloads, sketch_dtype="f32",
                 ranks=None, S0=None, steps_host=None, inputs=None):
        from concurrent.futures import ThreadPoolExecutor
        self.cfg, self.torch, self.ssm, self.wl = cfg, torch, ssm, workloads
        self.dev, self.W, self.U = dev, cfg.window, cfg.units
        self.sketch_dtype, self.ranks = sketch_dtype, ranks
        t0 = time.time()
        with ThreadPoolExecutor(8) as ex:
            if S0 is None:
                S0 = np.concatenate(list(ex.map(lambda n: workloads.initial_state(cfg, [n]),
                                                range(cfg.batch))))
            if steps_host is None:
                steps_host = list(ex.map(lambda t: workloads.step_inputs(cfg, t), range(n_steps)))
        self.S0, self.steps_host = S0, steps_host
        self.S0_dev = self.to_dev(S0) if not isinstance(S0, torch.Tensor) else S0
        self.inputs = inputs if inputs is not None else [
            tuple(self.to_dev(x) for x in (s.q, s.k, s.v, s.decay, s.beta)) for s in steps_host]
        self.gen_s = time.time() - t0
        P = lambda x: None if x is None else x.data_ptr()
        self.ptrs = [tuple(P(x) for x in step) for step in self.inputs]
        self.d = ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k, cfg.d_v,
                               cfg.window, cfg.rank, sketch_dtype)
        if ranks is not None:
            self.basis = self.to_dev(workloads.basis_ranked(cfg, ranks))
            self.offsets = ssm.rank_offsets(ranks)
            self.d_r = ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k,
                                     cfg.d_v, cfg.window, max(ranks), sketch_dtype)
        else:
            self.basis = self.to_dev(workloads.basis(cfg))
        W = self.W
        tin = torch.bfloat16 if cfg.in_dtype == "bf16" else torch.float32
        self.bufs = (torch.zeros((cfg.batch, cfg.heads, W, cfg.d_k), device=dev, dtype=tin),
                     torch.zeros((cfg.batch, cfg.heads, W, cfg.d_v), device=dev, dtype=tin),
                     torch.zeros(workloads.decay_shape(cfg, (cfg.batch, cfg.heads, W)), device=dev),
                     torch.zeros((cfg.batch, cfg.heads, W), device=dev) if cfg.has_beta else None)
        self.kb, self.vb, self.db, self.bb = (P(x) for x in self.bufs)
        self.y = torch.empty((cfg.batch, cfg.heads, cfg.d_v), device=dev)
        self.yp, self.bp = P(self.y), P(self.basis)
        self.stream = torch.cuda.current_stream()
        self.sp = self.stream.cuda_stream
        self.sk_rows = cfg.heads * cfg.rank if ranks is None else sum(ranks)
        self.sk_torch_dtype = torch.bfloat16 if sketch_dtype == "bf16" else torch.float32
        self.rmaps = {}  # sketch address -> its read map (least squares)
        self.coefficients("projection")

    def to_dev(self, x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            return self.torch.from_numpy(x.view(np.int16)).to(self.dev).view(self.torch.bfloat16)
        return self.torch.from_numpy(np.ascontiguousarray(x)).to(self.dev)

    # ---- the entry points of the chosen coefficient kind / rank policy ----------------
    def coefficients(self, kind: str) -> None:
        ssm, d = self.ssm, self.d
        _addr = lambda x: x if isinstance(x, int) else x.data_ptr()
        self.ls = kind == "least_squares"
        if self.ls:
            self.sketch_step = lambda sk, b, *x, **kw: ssm.sketch_decode_step_ls(
                d, sk, self.rmaps[_addr(sk)], *x, **kw)
            self.update_refresh = lambda st, sk, b, *x, **kw: ssm.window_update_refresh_ls(
                d, st, sk, self.rmaps[_addr(sk)], b, *x, **kw)
        elif self.ranks is None:
            self.sketch_step = lambda *x, **kw: ssm.sketch_decode_step(d, *x, **kw)
            self.update_refresh = lambda *x, **kw: ssm.window_update_refresh(d, *x, **kw)
        else:
            self.sketch_step = lambda *x, **kw: ssm.sketch_decode_step_ranked(
                self.d_r, self.offsets, *x, **kw)
            self.update_refresh = lambda *x, **kw: ssm.window_update_refresh_ranked(
                self.d_r, self.offsets, *x, **kw)

    def new_sketch(self):
        """A sketch array (and, for least squares, its read map) for the current kind."""
        cfg = self.cfg
        sk = self.torch.empty((cfg.batch, self.sk_rows, cfg.d_v), device=self.dev,
                              dtype=self.sk_torch_dtype)
        if self.ls:
            rm = self.torch.empty((cfg.batch, cfg.heads, cfg.rank, cfg.d_k), device=self.dev)
            self.rmaps[sk.data_ptr()] = rm.data_ptr()
            sk._read_map = rm  # keeps the map alive with the sketch
        return sk

    # ---- the legs ---------------------------------------------------------------------
    def run_sketch(self, state_p, sketch_p, t_lo, t_hi, sp, upd_events=None, only=None):
        """Sketch path: fused append + sketch read per step, update + refresh per window."""
        W, torch = self.W, self.torch
        for t in range(t_lo, t_hi):
            q, k, v, dc, b = self.ptrs[t]
            tau = t % W + 1
            if only in (None, "sketch"):
                self.sketch_step(sketch_p, self.bp, q, self.kb, self.vb, self.db, self.bb, tau,
                                 self.yp, k_t=k, v_t=v, decay_t=dc, beta_t=b, stream=sp)
            elif only == "update":  # keep the buffer fed without the read
                self.ssm.buffer_append(self.d, k, v, dc, b, self.kb, self.vb, self.db, self.bb,
                                       tau - 1, stream=sp)
            if tau == W and only in (None, "update"):
                if upd_events is not None:
                    upd_events.append((torch.cuda.Event(enable_timing=True),
                                       torch.cuda.Event(enable_timing=True)))
                    upd_events[-1][0].record(self.stream)
                self.update_refresh(state_p, sketch_p, self.bp, self.kb, self.vb, self.db,
                                    self.bb, W, stream=sp)
                if upd_events is not None:
                    upd_events[-1][1].record(self.stream)

    def run_full(self, state_p, t_lo, t_hi, sp, upd_events=None):
        """Exact buffered path: fused append + full-state read per step, update per window."""
        W, torch, ssm = self.W, self.torch, self.ssm
        for t in range(t_lo, t_hi):
            q, k, v, dc, b = self.ptrs[t]
            tau = t % W + 1
            ssm.full_read_decode_step(self.d, state_p, q, self.kb, self.vb, self.db, self.bb, tau,
                                      self.yp, k_t=k, v_t=v, decay_t=dc, beta_t=b, stream=sp)
            if tau == W:
                if upd_events is not None:
                    upd_events.append((torch.cuda.Event(enable_timing=True),
                                       torch.cuda.Event(enable_timing=True)))
                    upd_events[-1][0].record(self.stream)
                ssm.window_update_refresh(self.d, state_p, None, None, self.kb, self.vb, self.db,
                                          self.bb, W, stream=sp)
                if upd_events is not None:
                    upd_events[-1][1].record(self.stream)

    def run_rec(self, state_p, t_lo, t_hi, sp):
        for t in range(t_lo, t_hi):
            q, k, v, dc, b = self.ptrs[t]
            self.ssm.recurrent_decode_step(self.d, state_p, q, k, v, dc, b, self.yp, stream=sp)

    def timed(self, fn):
        torch = self.torch
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(self.stream)
        fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return max(e0.elapsed_time(e1) / 1e3, wall)

    def eager_timed(self, warm, run):
        """The eager legs: warm() enqueued, then run() right behind it with no host
        synchronisation between them, so that the device does not idle (and slow its first
        timed launches) between the warmup and the timed steps. Returns the HIP-event time
        of run() on the bench stream."""
        torch = self.torch
        torch.cuda.synchronize()
        warm()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        run()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    def graph_timed(self, enqueue):
        """Capture the timed steps into one HIP graph, replay once untimed, then time a replay."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(self.stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            enqueue(cap.cuda_stream)
        torch.cuda.synchronize()
        g.replay()
        t = self.timed(g.replay)
        del g
        return t

    def kernel_time(self, launch, reps):
        """Mean HIP-event time of `reps` launches on the bench stream (the first, untimed
        launch of a kernel in a process also loads its code)."""
        torch = self.torch
        launch(0)
        torch.cuda.synchronize()
        evs = []
        for i in range(reps):
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record(self.stream)
            launch(i)
            e_.record(self.stream)
            evs.append((s_, e_))
        torch.cuda.synchronize()
        return float(np.mean([s_.elapsed_time(e_) for s_, e_ in evs]))

    def sketch_path(self, warmup, total, only=None):
        """The sketch path from S0: eager (update events for the roofline), then as a graph.
        Returns (graph seconds, eager seconds, update launch ms list, state, sketch)."""
        state = self.S0_dev.clone()
        sketch = self.new_sketch()
        st_p, sk_p = state.data_ptr(), sketch.data_ptr()
        self.update_refresh(st_p, sk_p, self.bp, None, None, None, None, 0, stream=self.sp)
        upd_ev = []
        eager_s = self.eager_timed(
            lambda: self.run_sketch(st_p, sk_p, 0, warmup, self.sp, only=only),
            lambda: self.run_sketch(st_p, sk_p, warmup, total, self.sp, upd_ev, only=only))
        upd_ms = [s_.elapsed_time(e_) for s_, e_ in upd_ev]
        if only is not None:
            return None, eager_s, upd_ms, state, sketch
        graph_s = self.graph_timed(lambda cs: self.run_sketch(st_p, sk_p, warmup, total, cs))
        return graph_s, eager_s, upd_ms, state, sketch

    def update_steady_ms(self, windows: int = 16) -> dict:
        """HIP-event times of the update + refresh launches of up to `windows` windows of the
        sketch path run back to back from S0, with no host synchronisation between them;
        the mean and median over the second half. A launch that starts after the device has
        been idle, or fed by host launches slower than it runs, can take up to ~20% longer
        (kernel trace at W = 16: 950 us against 790 us)."""
        W = self.W
        n = min(windows, len(self.ptrs) // W)
        state = self.S0_dev.clone()
        sketch = self.new_sketch()
        st_p, sk_p = state.data_ptr(), sketch.data_ptr()
        self.update_refresh(st_p, sk_p, self.bp, None, None, None, None, 0, stream=self.sp)
        ev = []
        self.run_sketch(st_p, sk_p, 0, n * W, self.sp, ev)
        self.torch.cuda.synchronize()
        ms = [s_.elapsed_time(e_) for s_, e_ in ev][n // 2:]
        del state, sketch
        return {"mean_ms": float(np.mean(ms)), "median_ms": float(np.median(ms)),
                "launches": len(ms)}

    def full_path(self, warmup, total):
        state_f = self.S0_dev.clone()
        sf_p = state_f.data_ptr()
        upd_f = []
        eager_f = self.eager_timed(lambda: self.run_full(sf_p, 0, warmup, self.sp),
                                   lambda: self.run_full(sf_p, warmup, total, self.sp, upd_f))
        graph_f = self.graph_timed(lambda cs: self.run_full(sf_p, warmup, total, cs))
        steps = total - warmup
        return {"steps_per_s": steps / graph_f, "ms_per_step": graph_f * 1e3 / steps,
                "eager_steps_per_s": steps / eager_f,
                "update_no_refresh_ms": float(np.mean([s_.elapsed_time(e_) for s_, e_ in upd_f]))}

    def approx_error(self, T: int, kinds=("projection", "least_squares")) -> dict:
        """Error of the sketch read against the exact read over T decode steps from S0
        (untimed). Every step: the fused append + projection read, then the least-squares
        read and the exact full read of the same buffered tokens; at each window end one
        update + refresh writes the state and the projection sketch, and a refresh-only
        least-squares pass (n_tokens = 0) stores that kind's sketch rows and read map from
        the same state. Per-vector squared norms stay on the device until the end."""
        torch, ssm, cfg, W, U = self.torch, self.ssm, self.cfg, self.W, self.U
        kinds = [k for k in kinds if k == "projection" or self.ranks is None]
        st = self.S0_dev.clone()
        d_pr = self.d_r if self.ranks is not None else self.d
        sk = torch.empty((cfg.batch, self.sk_rows, cfg.d_v), device=self.dev,
                         dtype=self.sk_torch_dtype)
        refresh_pr = (lambda n, *b: ssm.window_update_refresh_ranked(
            d_pr, self.offsets, st, sk, self.basis, *b, n)) if self.ranks is not None else (
            lambda n, *b: ssm.window_update_refresh(d_pr, st, sk, self.basis, *b, n))
        read_pr = (lambda q, tau, y, **tok: ssm.sketch_decode_step_ranked(
            d_pr, self.offsets, sk, self.basis, q, *self.bufs, tau, y, **tok)) \
            if self.ranks is not None else (lambda q, tau, y, **tok: ssm.sketch_decode_step(
                d_pr, sk, self.basis, q, *self.bufs, tau, y, **tok))
        ls = "least_squares" in kinds
        if ls:  # the least-squares sketch rows are always fp32
            d_ls = ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k, cfg.d_v,
                                 W, cfg.rank, "f32")
            sk_q = torch.empty((cfg.batch, cfg.heads, cfg.rank, cfg.d_v), device=self.dev)
            rmap = torch.empty((cfg.batch, cfg.heads, cfg.rank, cfg.d_k), device=self.dev)

            def refresh_ls():
                ssm.window_update_refresh_ls(d_ls, st, sk_q, rmap, self.basis, None, None, None,
                                             None, 0)
        refresh_pr(0, None, None, None, None)
        if ls:
            refresh_ls()
        y_pr, y_ls, y_ex = (torch.empty_like(self.y) for _ in range(3))
        acc = {k: ([], []) for k in kinds}
        for t in range(T):
            q, k, v, dc, b = self.inputs[t]
            tau = t % W + 1
            read_pr(q, tau, y_pr, k_t=k, v_t=v, decay_t=dc, beta_t=b)
            if ls:
                ssm.sketch_decode_step_ls(d_ls, sk_q, rmap, q, *self.bufs, tau, y_ls)
            ssm.full_read_decode_step(self.d, st, q, *self.bufs, tau, y_ex)
            den = y_ex.view(U, -1).double().pow(2).sum(dim=1)
            for kind, yk in (("projection", y_pr), ("least_squares", y_ls)):
                if kind in acc:
                    acc[kind][0].append((yk - y_ex).view(U, -1).double().pow(2).sum(dim=1))
                    acc[kind][1].append(den)
            if tau == W:
                refresh_pr(W, *self.bufs)
                if ls:
                    refresh_ls()
        torch.cuda.synchronize()
        out = {"steps": T, "from": "initial state"}
        for kind, (num, den) in acc.items():
            out[kind] = error_summary(torch.stack(num).cpu().numpy(),
                                      torch.stack(den).cpu().numpy())
        return out


def read_traffic_file(cfg, same_workload: bool):
    """HBM bytes per update launch from the committed counter runs, if they were taken on
    this kernel source and this workload."""
    if not os.path.exists(TRAFFIC_FILE) or not same_workload:
        return None
    tr = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            key, sep, val = line.strip().partition(": ")
            if sep and key in ("config", "kernel_source_hash", "bytes_per_launch"):
                tr[key] = val
    if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("config") == cfg.name:
        return float(tr["bytes_per_launch"])
    return None


def sweep_c5(a, torch, ssm, workloads, dev) -> int:
    """The GDN sweep: N=1024, H=32, 128 x 128 state; r in {4, 8, 16, 32} x W in {4, 8, 16}.
    The 12 points share one token stream and one initial state (generated once); only the
    basis follows the rank and the window buffer the window. Each point times the sketch
    path and the exact full-read path on the same tokens (HIP graphs, whole windows), the
    update + refresh launches (HIP events), and reports the approximation error over T."""
    base = workloads.c5(8, 8)
    T = base.steps
    # at least 8 update launches at every point: one launch's time moves by up to ~10% with
    # what the caches hold when it starts (kernel trace at W = 16: 788 to 936 us)
    # and at least 4 windows of warmup: after the device has been idle, memory-bound launches
    # run slow for a few milliseconds (the first W = 16 updates up to ~20%)
    w_max = max(workloads.C5_WINDOWS)
    steps, warmup = plan_steps(max(a.steps, 8 * w_max), max(a.warmup, 4 * w_max), w_max)
    n_steps = max(T, steps + warmup)
    shared = None
    for W in workloads.C5_WINDOWS:
        for r in workloads.C5_RANKS:
            cfg = workloads.c5(r, W)
            w0 = time.time()
            if shared is None:
                L = Layer(cfg, n_steps, dev, torch, ssm, workloads)
                shared = dict(S0=L.S0_dev, steps_host=L.steps_host, inputs=L.inputs)
                # the per-token decode (every step writes and reads the full state) does not
                # depend on r or W: timed once, on the same tokens, as the points' comparator
                state_r = L.S0_dev.clone()
                sr_p = state_r.data_ptr()
                L.run_rec(sr_p, 0, warmup, L.sp)
                per_token_sps = steps / L.graph_timed(lambda cs: L.run_rec(sr_p, warmup,
                                                                           warmup + steps, cs))
                del state_r
            else:
                L = Layer(cfg, n_steps, dev, torch, ssm, workloads, **shared)
            total = warmup + steps
            graph_s, eager_s, upd_ms, st, sk = L.sketch_path(warmup, total)
            del st, sk
            full = L.full_path(warmup, total)
            bm = bytes_model(cfg)
            U = cfg.units
            upd_avg = float(np.mean(upd_ms))
            upd_gbs = bm["update"] * U / (upd_avg * 1e-3) / 1e9
            steady = L.update_steady_ms()
            steady_gbs = bm["update"] * U / (steady["mean_ms"] * 1e-3) / 1e9
            tau_mid = W // 2 + 1
            q0 = L.ptrs[0][0]
            state_probe = L.S0_dev.clone()
            sk_probe = L.new_sketch()
            L.update_refresh(state_probe.data_ptr(), sk_probe.data_ptr(), L.bp, None, None, None,
                             None, 0, stream=L.sp)
            sk_ms = L.kernel_time(lambda i: L.sketch_step(
                sk_probe.data_ptr(), L.bp, q0, L.kb, L.vb, L.db, L.bb, tau_mid, L.yp,
                stream=L.sp), 20)
            full_ms = L.kernel_time(lambda i: ssm.full_read_decode_step(
                L.d, state_probe.data_ptr(), q0, L.kb, L.vb, L.db, L.bb, tau_mid, L.yp,
                stream=L.sp), 10)
            del state_probe, sk_probe
            approx = L.approx_error(T)
            value = steps / graph_s
            print(json.dumps({
                "sweep": "c5", "point": cfg.name, "rank": r, "window": W,
                "workload": cfg.description, "steps": steps, "warmup": warmup,
                "steps_per_s": value, "ms_per_step": graph_s * 1e3 / steps,
                "eager_steps_per_s": steps / eager_s,
                "full_read_steps_per_s": full["steps_per_s"],
                "speedup_vs_full_read": value / full["steps_per_s"],
                "per_token_steps_per_s": per_token_sps,
                "speedup_vs_per_token": value / per_token_sps,
                "update_refresh_ms": upd_avg, "update_refresh_gbs": upd_gbs,
                "update_refresh_ms_median": float(np.median(upd_ms)),
                "update_launches": len(upd_ms),
                "update_refresh_steady": dict(steady, gbs=steady_gbs,
                                              frac=steady_gbs / HBM_PEAK_GBS),
                "update_refresh_frac": upd_gbs / HBM_PEAK_GBS,
                "update_no_refresh_ms": full["update_no_refresh_ms"],
                "sketch_decode_ms_tau_mid": sk_ms, "full_read_decode_ms_tau_mid": full_ms,
                "tau_mid": tau_mid,
                "state_bytes_per_step": {"sketch": bm["state_bytes_sketch"],
                                         "full": bm["state_bytes_full"],
                                         "ratio": bm["state_bytes_full"] / bm["state_bytes_sketch"]},
                "read_path_bytes_ratio": bm["full_step"] / bm["sketch_step"],
                "amortized_bytes_ratio": bm["amortized_full"] / bm["amortized_sketch"],
                "approx_error": approx, "point_wall_s": time.time() - w0}), flush=True)
            del L
            torch.cuda.empty_cache()
    return 0


def parse_args(argv=None) -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64,
                    help="timed decode steps (rounded up to whole windows)")
    ap.add_argument("--warmup", type=int, default=16,
                    help="untimed decode steps first (rounded up to whole windows)")
    ap.add_argument("--config", default="c3")
    ap.add_argument("--sweep", choices=["c5"], default=None,
                    help="c5: the 12 (r, W) points of the GDN sweep, one JSON line each")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true", help="skip the full-read comparison pass")
    ap.add_argument("--fit-basis", action="store_true",
                    help="fit the basis on the device (ssm_fit_basis) from the workload's sampled "
                         "queries instead of taking the host one; reports the fit's time")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache (Infinity Cache flushed) kernel timings")
    ap.add_argument("--cpu-units", type=int, default=512, help="oracle sample: units")
    ap.add_argument("--cpu-steps", type=int, default=16, help="oracle sample: decode steps")
    ap.add_argument("--only", choices=["sketch", "full", "update"], default=None,
                    help="profiling: run only this leg's launches")
    ap.add_argument("--schedule", choices=["lockstep", "staggered"], default="lockstep",
                    help="staggered: sequence n sits at window position n mod W, so every step "
                         "updates N/W sequences (variable-length entry points, slot map)")
    ap.add_argument("--per-head-ranks", choices=["avg8"], default=None,
                    help="per-head sketch ranks (avg8: 2, 4, 8, 18 cycled over heads, mean 8)")
    ap.add_argument("--sketch-dtype", choices=["f32", "bf16"], default="f32",
                    help="storage type of the sketch (the headline workload keeps fp32)")
    ap.add_argument("--coefficients", choices=["projection", "least_squares"],
                    default="projection", help="sketch-read coefficients (headline: projection)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="profiling: copy MIB MiB with a plain device copy kernel, then exit")
    return ap.parse_args(argv)


def main(argv=None) -> int:
    a = parse_args(argv)
    wall0 = time.time()

    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (the decode path "
              "shards by whole heads or sequences with no exchange step).", file=sys.stderr)
        return 2

    import torch
    import workloads
    import sketched_recurrent_state_amd as ssm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")

    if a.copy_calibration:
        n = a.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))
        return 0

    if a.sweep == "c5":
        return sweep_c5(a, torch, ssm, workloads, dev)

    cfg = workloads.get(a.config)
    W = cfg.window
    steps, warmup = plan_steps(a.steps, a.warmup, W)
    total = warmup + steps
    U = cfg.units
    ranks = workloads.average_rank_8(cfg.heads) if a.per_head_ranks == "avg8" else None
    ls = a.coefficients == "least_squares"
    if ls and (ranks is not None or a.schedule != "lockstep" or a.sketch_dtype != "f32"):
        print("least-squares coefficients run with uniform ranks, lockstep and an fp32 sketch",
              file=sys.stderr)
        return 2
    if a.fit_basis and ranks is not None:
        print("--fit-basis fits one uniform rank", file=sys.stderr)
        return 2

    # ---- inputs, resident in HBM before timing (the approximation pass needs T steps) ----
    L = Layer(cfg, max(total, cfg.steps), dev, torch, ssm, workloads, a.sketch_dtype, ranks)
    basis_fit = None
    if a.fit_basis:
        # the basis fitted on the device from the workload's sampled queries (4096 per head)
        # replaces the host one for every GPU leg; timed once warm, outside the timed region
        d_fit = ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k, cfg.d_v, W,
                              cfg.rank)
        samples = L.to_dev(workloads.pca_samples(cfg))
        n_fit = samples.shape[1]
        ssm.fit_basis(d_fit, samples, n_fit, L.basis)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(3):
            ssm.fit_basis(d_fit, samples, n_fit, L.basis)
        ev[1].record()
        torch.cuda.synchronize()
        basis_fit = {"ms": ev[0].elapsed_time(ev[1]) / 3, "samples_per_head": n_fit,
                     "heads": cfg.heads, "rank": cfg.rank}
        del samples
    L.coefficients(a.coefficients)
    sp, P = L.sp, (lambda x: None if x is None else x.data_ptr())
    kb, vb, db, bb, yp, bp = L.kb, L.vb, L.db, L.bb, L.yp, L.bp
    bm = bytes_model(cfg, 2 if a.sketch_dtype == "bf16" else 4, ls)

    # ---- the sketch path: eager launches (update kernel timed by HIP events), then the
    # same steps as one HIP graph (headline) ---------------------------------------------
    elapsed, eager_s, upd_ms, state, sketch = L.sketch_path(warmup, total, only=a.only)
    if a.only is not None:  # profiling runs stop here
        print(json.dumps({"only": a.only, "steps": steps, "warmup": warmup,
                          "ms_per_step": eager_s * 1e3 / steps}))
        return 0
    st_p, sk_p = P(state), P(sketch)

    # ---- staggered windows (serving shape): every step updates N/W sequences -----------
    # Sequence n sits at window position n mod W. Headline of this leg: one
    # ssm_decode_step_varlen launch per step (the read of every row and the update of the
    # rows whose window fills, the sketch double-buffered per row); beside it the same
    # schedule as two launches per step (a varlen read, then a varlen update).
    staggered = None
    if a.schedule == "staggered":
        N = cfg.batch
        d = L.d
        i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)
        taus = [i32([((ph + n) % W) + 1 for n in range(N)]) for ph in range(W)]
        ups = [i32([n for n in range(N) if ((ph + n) % W) + 1 == W]) for ph in range(W)]
        pars = [i32([((t + n) // W) % 2 for n in range(N)]) for t in range(2 * W)]
        fulls = [torch.full((len(u),), W, dtype=torch.int32, device=dev) for u in ups]
        d_ups = [ssm.Dims.make(cfg.rule, cfg.in_dtype, len(u), cfg.heads, cfg.d_k, cfg.d_v, W,
                               cfg.rank, a.sketch_dtype) for u in ups]
        tp, up, fp, pp = ([P(x) for x in taus], [P(x) for x in ups], [P(x) for x in fulls],
                          [P(x) for x in pars])
        sketch_alt = L.new_sketch()
        ska_p = P(sketch_alt)
        L.update_refresh(st_p, ska_p, bp, None, None, None, None, 0, stream=sp)

        def run_single(t_lo, t_hi, sp_):
            for t in range(t_lo, t_hi):
                q, k, v, dc, b = L.ptrs[t]
                ph = t % W
                ssm.decode_step_varlen(d, N, None, tp[ph], pp[t % (2 * W)], d_ups[ph].batch,
                                       up[ph], st_p, sk_p, ska_p, bp, q, k, v, dc, b, kb, vb, db,
                                       bb, yp, stream=sp_)

        def run_two(t_lo, t_hi, sp_, upd_events=None):
            for t in range(t_lo, t_hi):
                q, k, v, dc, b = L.ptrs[t]
                ph = t % W
                ssm.sketch_decode_step_varlen(d, N, None, tp[ph], sk_p, bp, q, kb, vb, db, bb, yp,
                                              k_t=k, v_t=v, decay_t=dc, beta_t=b, stream=sp_)
                if d_ups[ph].batch:
                    if upd_events is not None:
                        upd_events.append((torch.cuda.Event(enable_timing=True),
                                           torch.cuda.Event(enable_timing=True)))
                        upd_events[-1][0].record(L.stream)
                    ssm.window_update_refresh_varlen(d_ups[ph], N, up[ph], fp[ph], st_p, sk_p, bp,
                                                     kb, vb, db, bb, stream=sp_)
                    if upd_events is not None:
                        upd_events[-1][1].record(L.stream)

        eager_1 = L.eager_timed(lambda: run_single(0, warmup, sp),
                                lambda: run_single(warmup, total, sp))
        graph_1 = L.graph_timed(lambda cs: run_single(warmup, total, cs))
        step_ms = L.kernel_time(lambda i: ssm.decode_step_varlen(
            d, N, None, tp[W - 1], pp[W - 1], d_ups[W - 1].batch, up[W - 1], st_p, sk_p, ska_p,
            bp, *L.ptrs[0][:5], kb, vb, db, bb, yp, stream=sp), 16)
        stg_ev = []
        eager_2 = L.eager_timed(lambda: run_two(0, warmup, sp),
                                lambda: run_two(warmup, total, sp, stg_ev))
        graph_2 = L.graph_timed(lambda cs: run_two(warmup, total, cs))
        staggered = {"steps_per_s": steps / graph_1, "ms_per_step": graph_1 * 1e3 / steps,
                     "eager_steps_per_s": steps / eager_1, "launch_ms": step_ms,
                     "entry_point": "ssm_decode_step_varlen (one launch per step)",
                     "two_launch": {"steps_per_s": steps / graph_2,
                                    "eager_steps_per_s": steps / eager_2,
                                    "update_per_step_ms": float(np.mean(
                                        [s_.elapsed_time(e_) for s_, e_ in stg_ev]))},
                     "sequences_updated_per_step": N / W,
                     "vs_lockstep": (steps / graph_1) / (steps / elapsed)}
        del sketch_alt

    # ---- per-kernel time of the sketch read and the full read (events around each launch) --
    tau_mid = W // 2 + 1
    # bytes of one read at window position tau_mid, the token already buffered (no append):
    # q + tau_mid buffered tokens + y, plus the sketch (and read map) or the full state
    s_in = 2 if cfg.in_dtype == "bf16" else 4
    common = cfg.d_k * s_in + tau_mid * bm["tok"] + 4 * cfg.d_v
    sk_b = U * (bm["state_bytes_sketch"] + (4 * cfg.rank * cfg.d_k if ls else 0) + common)
    full_b = U * (bm["state_bytes_full"] + common)
    q0 = L.ptrs[0][0]
    sketch_ms = L.kernel_time(lambda i: L.sketch_step(sk_p, bp, q0, kb, vb, db, bb, tau_mid, yp,
                                                      stream=sp), 20)
    full_ms = L.kernel_time(lambda i: ssm.full_read_decode_step(L.d, st_p, q0, kb, vb, db, bb,
                                                                tau_mid, yp, stream=sp), 10)

    # ---- the exact full-read path on the same tokens (comparison) ----------------------
    full = None if a.no_compare else L.full_path(warmup, total)

    # ---- the per-token recurrent decode (the standard baseline) on the same tokens -----
    per_token = None
    if not a.no_compare:
        state_r = L.S0_dev.clone()
        sr_p = P(state_r)
        eager_r = L.eager_timed(lambda: L.run_rec(sr_p, 0, warmup, sp),
                                lambda: L.run_rec(sr_p, warmup, total, sp))
        graph_r = L.graph_timed(lambda cs: L.run_rec(sr_p, warmup, total, cs))
        q0_, k0_, v0_, d0_, b0_ = L.ptrs[0]
        rec_ms = L.kernel_time(lambda i: ssm.recurrent_decode_step(L.d, sr_p, q0_, k0_, v0_, d0_,
                                                                   b0_, yp, stream=sp), 10)
        rec_bytes = U * (8 * cfg.d_k * cfg.d_v + bm["tok"] + cfg.d_k * s_in + 4 * cfg.d_v)
        per_token = {"steps_per_s": steps / graph_r, "ms_per_step": graph_r * 1e3 / steps,
                     "eager_steps_per_s": steps / eager_r, "kernel_ms": rec_ms,
                     "kernel_gbs": rec_bytes / (rec_ms * 1e-3) / 1e9}
        del state_r

    # ---- approximation error of the sketch read vs the exact read over T steps (untimed) --
    approx = L.approx_error(cfg.steps)

    # ---- attainable HBM rate: a plain device copy of 2 GiB (read + write) ---------------
    n_copy = (2 << 30) // 4
    src = torch.ones(n_copy, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = L.kernel_time(lambda i: dst.copy_(src), 5)
    copy_gbs = 2 * n_copy * 4 / (copy_ms * 1e-3) / 1e9
    del src, dst

    # ---- attainable HBM rate for the state's read + write: the library's in-place stream
    # probe over a buffer of the state's size, in the update's access order (shape 0) and in
    # flat 128 KB runs per workgroup (shape 1, the fastest plain shape measured) -----------
    n_tiles = max(2, (L.S0_dev.numel() * 4 // 65536) & ~1)  # at least two tiles (tiny configs)
    n_small = max(2, int(round(sk_b / 2 / 65536)) & ~1)
    probe = torch.ones(max(n_tiles, n_small) * 16384, device=dev)
    probe_gbs = []
    for shape in (0, 1):
        ms = L.kernel_time(lambda i: ssm.stream_probe(probe[:n_tiles * 16384], n_tiles, shape,
                                                      stream=sp), 10)
        probe_gbs.append(2 * n_tiles * 65536 / (ms * 1e-3) / 1e9)
    # and over a buffer whose read + write equals one sketch read's bytes: the ceiling of a
    # single short streaming launch of that size, launch and ramp included
    small = probe[:n_small * 16384]
    small_ms = L.kernel_time(lambda i: ssm.stream_probe(small, n_small, 1, stream=sp), 20)
    del probe, small
    stream_probe = {"bytes_each_way": n_tiles * 65536, "launches": 10,
                    "update_order_gbs": probe_gbs[0], "flat_runs_gbs": probe_gbs[1],
                    "sketch_size_bytes": 2 * n_small * 65536,
                    "sketch_size_gbs": 2 * n_small * 65536 / (small_ms * 1e-3) / 1e9}

    # ---- cold-cache kernel times: the 256 MB Infinity Cache flushed before each launch ----
    # A 512 MiB read between launches, outside the events, replaces the cached lines with
    # clean ones. (A write would leave them dirty, and the timed kernel would pay for their
    # write-back.) Without a flush, part of the sketch step's working set, and of the state
    # the previous update wrote, is served from that cache.
    cold = None
    if not a.no_cold:
        flush = torch.ones((512 << 20) // 4, device=dev)
        flush_sum = torch.empty((), device=dev)
        st_c, sk_c = L.S0_dev.clone(), L.new_sketch()
        L.update_refresh(st_c, sk_c, L.basis, None, None, None, None, 0, stream=L.stream)

        def cold_time(launch, reps=5):
            evs = []
            launch()
            for i in range(reps):
                torch.sum(flush, dim=0, out=flush_sum)
                s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s_.record(L.stream)
                launch()
                e_.record(L.stream)
                evs.append((s_, e_))
            torch.cuda.synchronize()
            return float(np.mean([s_.elapsed_time(e_) for s_, e_ in evs]))

        stc_p, skc_p = P(st_c), P(sk_c)
        c_upd = cold_time(lambda: L.update_refresh(stc_p, skc_p, bp, kb, vb, db, bb, W, stream=sp))
        c_sk = cold_time(lambda: L.sketch_step(skc_p, bp, q0, kb, vb, db, bb, tau_mid, yp, stream=sp))
        c_full = cold_time(lambda: ssm.full_read_decode_step(L.d, stc_p, q0, kb, vb, db, bb,
                                                             tau_mid, yp, stream=sp))
        cold = {"flush_bytes": flush.numel() * 4, "tau": tau_mid,
                "update_refresh_ms": c_upd, "update_refresh_gbs": bm["update"] * U / (c_upd * 1e-3) / 1e9,
                "sketch_decode_ms": c_sk, "sketch_decode_gbs": sk_b / (c_sk * 1e-3) / 1e9,
                "full_read_decode_ms": c_full, "full_read_decode_gbs": full_b / (c_full * 1e-3) / 1e9}
        for key in ("update_refresh", "sketch_decode", "full_read_decode"):
            cold[key + "_frac"] = cold[key + "_gbs"] / HBM_PEAK_GBS
        del flush, flush_sum, st_c, sk_c

    # ---- roofline of the dominant kernel (update + refresh) ---------------------------
    upd_avg_ms = float(np.mean(upd_ms))
    upd_bytes = bm["update"] * U
    achieved = upd_bytes / (upd_avg_ms * 1e-3) / 1e9
    # counters describe the lockstep, uniform-rank, fp32-sketch decode of their workload
    traffic = read_traffic_file(cfg, a.schedule == "lockstep" and ranks is None
                                and a.sketch_dtype == "f32" and not ls)

    # ---- CPU baseline: the oracle on a bounded sample --------------------------------
    cpu = None
    if not a.no_cpu_baseline:
        import oracle
        units = workloads.sample_units(cfg, min(a.cpu_units, U))
        Ts = min(a.cpu_steps, len(L.steps_host))
        flat = lambda x, e: x.reshape((U,) + ((e,) if e else ()))[units]
        h = [L.steps_host[t] for t in range(Ts)]
        q = np.stack([workloads.widen(flat(s.q, cfg.d_k)) for s in h])
        k = np.stack([workloads.widen(flat(s.k, cfg.d_k)) for s in h])
        v = np.stack([workloads.widen(flat(s.v, cfg.d_v)) for s in h])
        dc = np.stack([flat(s.decay, cfg.d_k if cfg.per_channel_decay else 0) for s in h]).astype(np.float64)
        be = (np.stack([flat(s.beta, 0) for s in h]).astype(np.float64) if cfg.has_beta else None)
        S0s = L.S0.reshape(U, cfg.d_k, cfg.d_v)[units].astype(np.float64)
        Bs = workloads.basis(cfg)[units % cfg.heads].astype(np.float64)
        threads = oracle.max_threads()
        c0 = time.perf_counter()
        oracle.run(cfg.rule, S0s, Bs, q, k, v, dc, be, W, threads=threads)
        cpu_s = time.perf_counter() - c0
        steps_per_s = Ts / (cpu_s * U / len(units))
        # one thread on the first 64 sampled units: the per-core rate
        n1 = min(64, len(units))
        c0 = time.perf_counter()
        oracle.run(cfg.rule, S0s[:n1], Bs[:n1], q[:, :n1], k[:, :n1], v[:, :n1], dc[:, :n1],
                   be[:, :n1] if be is not None else None, W, threads=1)
        one_s = time.perf_counter() - c0
        cpu = {"value": steps_per_s, "unit": "decode steps/s", "cores": threads, "kind": "oracle",
               "sample": f"{len(units)} of {U} (sequence, head) units x {Ts} steps, fp64, "
                         f"{cpu_s:.2f} s wall on {threads} threads; rate scaled to all {U} units",
               "cpu_model": cpu_model(),
               "one_thread": {"value": Ts / (one_s * U / n1), "unit": "decode steps/s",
                              "sample": f"{n1} units x {Ts} steps on 1 thread, {one_s:.2f} s; "
                                        f"rate scaled to all {U} units"}}

    value = steps / elapsed
    out = {
        "metric": metric_name(cfg),
        "value": value,
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "steps_requested": a.steps,
        "warmup_requested": a.warmup,
        "ms_per_step": elapsed * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.description, "rule": cfg.rule, "batch": cfg.batch,
                   "heads": cfg.heads, "d_k": cfg.d_k, "d_v": cfg.d_v, "window": W,
                   "rank": cfg.rank if ranks is None else f"per head {sorted(set(ranks))}, mean "
                   f"{sum(ranks) / len(ranks):g}", "inputs": cfg.in_dtype, "state": "f32",
                   "sketch": a.sketch_dtype, "coefficients": a.coefficients,
                   "schedule": a.schedule, "basis": "device fit" if a.fit_basis else "host"},
        "roofline": {"bound": "hbm", "kernel": "update_refresh_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "bytes_per_launch": upd_bytes,
                     "avg_launch_ms": upd_avg_ms, "launches": len(upd_ms)},
        "cpu_baseline": cpu,
        "tokens_per_s": value * cfg.batch,
        "kernels_ms": {"update_refresh": upd_avg_ms, "sketch_decode": sketch_ms,
                       "full_read_decode": full_ms},
        "sketch_decode_gbs": sk_b / (sketch_ms * 1e-3) / 1e9,
        "full_read_decode_gbs": full_b / (full_ms * 1e-3) / 1e9,
        "sketch_read_frac_of_stream": (sk_b / (sketch_ms * 1e-3) / 1e9) / stream_probe["sketch_size_gbs"],
        "eager_steps_per_s": steps / eager_s,
        "full_read_path": full,
        "speedup_vs_full_read": (value / full["steps_per_s"]) if full else None,
        "per_token_path": per_token,
        "staggered_windows": staggered,
        "speedup_vs_per_token": (value / per_token["steps_per_s"]) if per_token else None,
        "bytes_per_unit": {k: bm[k] for k in ("state_bytes_sketch", "state_bytes_full", "sketch_step",
                                              "full_step", "amortized_sketch", "amortized_full")},
        "state_bytes_ratio": bm["state_bytes_full"] / bm["state_bytes_sketch"],
        "read_path_bytes_ratio": bm["full_step"] / bm["sketch_step"],
        "approx_error": approx,
        "cold_cache": cold,
        "basis_fit": basis_fit,
        "copy_probe_gbs": copy_gbs,
        "update_refresh_frac_of_copy": achieved / copy_gbs,
        "stream_probe": stream_probe,
        "update_refresh_frac_of_stream": achieved / max(probe_gbs),
        "input_gen_s": L.gen_s,
        "bench_wall_s": time.time() - wall0,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
