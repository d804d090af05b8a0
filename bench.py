#!/usr/bin/env python3
"""Decode-throughput benchmark of the SketchSSM windowed decode path on one GPU.

Workload (default): a Gated DeltaNet decode layer, N=256 sequences x H=32
heads, 128 x 128 fp32 state per (sequence, head), bf16 q/k/v, window W=8,
sketch rank r=8. One timed step is one decode step of the whole layer: the
current token is appended to the window buffer and the output is read from
the sketch (one fused launch); after every W-th step the fused update +
refresh writes the state once and stores the new sketch. K must be a multiple
of W so that every window's state write is inside the timed region. The K
timed steps are captured once into a HIP graph and the headline times one
replay of it; the same steps launched one by one are timed too (eager), with
HIP events around every update + refresh launch for the roofline.

Prints one JSON line. Extra fields: per-kernel times, two comparison paths on
the same tokens (the exact buffered full read, and the per-token recurrent
decode that updates and reads the whole state every step), the byte model,
the sketch's approximation error, and the oracle's CPU rate on a bounded
sample.

    python bench.py [--steps 64] [--warmup 16] [--config c3]
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
KERNEL_SOURCES = ["common.hpp", "update_refresh.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, "sketched_recurrent_state_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="c3")
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
    a = ap.parse_args()

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

    cfg = workloads.get(a.config)
    W = cfg.window
    if a.steps % W or a.warmup % W:
        print(f"--steps and --warmup must be multiples of the window W={W}", file=sys.stderr)
        return 2
    total = a.warmup + a.steps
    d = ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k, cfg.d_v, W, cfg.rank,
                      a.sketch_dtype)
    U = cfg.units

    # ---- inputs, resident in HBM before timing ---------------------------------------
    from concurrent.futures import ThreadPoolExecutor

    def to_dev(x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    t0 = time.time()
    with ThreadPoolExecutor(8) as ex:
        S0 = np.concatenate(list(ex.map(lambda n: workloads.initial_state(cfg, [n]), range(cfg.batch))))
        steps_host = list(ex.map(lambda t: workloads.step_inputs(cfg, t), range(total)))
    S0_dev = to_dev(S0)
    ranks = workloads.average_rank_8(cfg.heads) if a.per_head_ranks == "avg8" else None
    if ranks is not None:
        basis = to_dev(workloads.basis_ranked(cfg, ranks))
        offsets = ssm.rank_offsets(ranks)
        d_r = ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k, cfg.d_v, W,
                            max(ranks), a.sketch_dtype)
    else:
        basis = to_dev(workloads.basis(cfg))
    basis_fit = None
    if a.fit_basis:
        # the basis fitted on the device from the workload's sampled queries (4096 per head)
        # replaces the host one for every GPU leg; timed once warm, outside the timed region
        if ranks is not None:
            print("--fit-basis fits one uniform rank", file=sys.stderr)
            return 2
        d_fit = ssm.Dims.make(cfg.rule, cfg.in_dtype, cfg.batch, cfg.heads, cfg.d_k, cfg.d_v, W,
                              cfg.rank)
        samples = to_dev(workloads.pca_samples(cfg))
        n_fit = samples.shape[1]
        ssm.fit_basis(d_fit, samples, n_fit, basis)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(3):
            ssm.fit_basis(d_fit, samples, n_fit, basis)
        ev[1].record()
        torch.cuda.synchronize()
        basis_fit = {"ms": ev[0].elapsed_time(ev[1]) / 3, "samples_per_head": n_fit,
                     "heads": cfg.heads, "rank": cfg.rank}
        del samples
    inputs = [(to_dev(s.q), to_dev(s.k), to_dev(s.v), to_dev(s.decay), to_dev(s.beta))
              for s in steps_host]
    gen_s = time.time() - t0

    tin = torch.bfloat16 if cfg.in_dtype == "bf16" else torch.float32
    k_buf = torch.zeros((cfg.batch, cfg.heads, W, cfg.d_k), device=dev, dtype=tin)
    v_buf = torch.zeros((cfg.batch, cfg.heads, W, cfg.d_v), device=dev, dtype=tin)
    d_buf = torch.zeros(workloads.decay_shape(cfg, (cfg.batch, cfg.heads, W)), device=dev)
    b_buf = torch.zeros((cfg.batch, cfg.heads, W), device=dev) if cfg.has_beta else None
    bufs = (k_buf, v_buf, d_buf, b_buf)
    y = torch.empty((cfg.batch, cfg.heads, cfg.d_v), device=dev)
    stream = torch.cuda.current_stream()

    # Raw device addresses: the timed loops go straight through the C ABI.
    P = lambda x: None if x is None else x.data_ptr()
    ptrs = [tuple(P(x) for x in step) for step in inputs]
    kb, vb, db, bb = (P(x) for x in bufs)
    yp, bp = P(y), P(basis)

    ls = a.coefficients == "least_squares"
    if ls and (ranks is not None or a.schedule != "lockstep" or a.sketch_dtype != "f32"):
        print("least-squares coefficients run with uniform ranks, lockstep and an fp32 sketch",
              file=sys.stderr)
        return 2
    rmaps = {}  # sketch address -> its read map (least squares)

    def _addr(x):
        return x if isinstance(x, int) else x.data_ptr()

    if ls:
        sketch_step = lambda sk, b, *x, **kw: ssm.sketch_decode_step_ls(
            d, sk, rmaps[_addr(sk)], *x, **kw)
        update_refresh = lambda st, sk, b, *x, **kw: ssm.window_update_refresh_ls(
            d, st, sk, rmaps[_addr(sk)], b, *x, **kw)
    elif ranks is None:
        sketch_step = lambda *x, **kw: ssm.sketch_decode_step(d, *x, **kw)
        update_refresh = lambda *x, **kw: ssm.window_update_refresh(d, *x, **kw)
    else:
        sketch_step = lambda *x, **kw: ssm.sketch_decode_step_ranked(d_r, offsets, *x, **kw)
        update_refresh = lambda *x, **kw: ssm.window_update_refresh_ranked(d_r, offsets, *x, **kw)

    def run_sketch(state_p, sketch_p, t_lo, t_hi, sp, upd_events=None, only=None):
        """Sketch path: fused append + sketch read per step, update + refresh per window."""
        for t in range(t_lo, t_hi):
            q, k, v, dc, b = ptrs[t]
            tau = t % W + 1
            if only in (None, "sketch"):
                sketch_step(sketch_p, bp, q, kb, vb, db, bb, tau, yp, k_t=k, v_t=v,
                            decay_t=dc, beta_t=b, stream=sp)
            elif only == "update":  # keep the buffer fed without the read
                ssm.buffer_append(d, k, v, dc, b, kb, vb, db, bb, tau - 1, stream=sp)
            if tau == W and only in (None, "update"):
                if upd_events is not None:
                    upd_events.append((torch.cuda.Event(enable_timing=True),
                                       torch.cuda.Event(enable_timing=True)))
                    upd_events[-1][0].record(stream)
                update_refresh(state_p, sketch_p, bp, kb, vb, db, bb, W, stream=sp)
                if upd_events is not None:
                    upd_events[-1][1].record(stream)

    def run_full(state_p, t_lo, t_hi, sp, upd_events=None):
        """Exact buffered path: fused append + full-state read per step, update per window."""
        for t in range(t_lo, t_hi):
            q, k, v, dc, b = ptrs[t]
            tau = t % W + 1
            ssm.full_read_decode_step(d, state_p, q, kb, vb, db, bb, tau, yp, k_t=k, v_t=v,
                                      decay_t=dc, beta_t=b, stream=sp)
            if tau == W:
                if upd_events is not None:
                    upd_events.append((torch.cuda.Event(enable_timing=True),
                                       torch.cuda.Event(enable_timing=True)))
                    upd_events[-1][0].record(stream)
                ssm.window_update_refresh(d, state_p, None, None, kb, vb, db, bb, W, stream=sp)
                if upd_events is not None:
                    upd_events[-1][1].record(stream)

    def timed(fn):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return max(e0.elapsed_time(e1) / 1e3, wall)

    def graph_timed(enqueue):
        """Capture the K timed steps into one HIP graph, replay once untimed, then time a replay."""
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            enqueue(cap.cuda_stream)
        torch.cuda.synchronize()
        g.replay()
        return timed(g.replay), g

    sp = stream.cuda_stream
    bm = bytes_model(cfg, 2 if a.sketch_dtype == "bf16" else 4, ls)

    # ---- the sketch path, eager launches (update kernel timed by HIP events) ---------
    state = S0_dev.clone()
    sk_rows = cfg.heads * cfg.rank if ranks is None else sum(ranks)
    sk_dtype = torch.bfloat16 if a.sketch_dtype == "bf16" else torch.float32
    sketch = torch.empty((cfg.batch, sk_rows, cfg.d_v), device=dev, dtype=sk_dtype)
    if ls:
        rm_main = torch.empty((cfg.batch, cfg.heads, cfg.rank, cfg.d_k), device=dev)
        rmaps[sketch.data_ptr()] = rm_main.data_ptr()
    st_p, sk_p = P(state), P(sketch)
    update_refresh(st_p, sk_p, bp, None, None, None, None, 0, stream=sp)
    run_sketch(st_p, sk_p, 0, a.warmup, sp, only=a.only)
    upd_ev = []
    eager_s = timed(lambda: run_sketch(st_p, sk_p, a.warmup, total, sp, upd_ev, only=a.only))
    upd_ms = [s_.elapsed_time(e_) for s_, e_ in upd_ev]

    if a.only is not None:  # profiling runs stop here
        print(json.dumps({"only": a.only, "steps": a.steps, "ms_per_step": eager_s * 1e3 / a.steps}))
        return 0

    # ---- the sketch path as one HIP graph (headline) -----------------------------------
    graph_s, g_sketch = graph_timed(lambda cs: run_sketch(st_p, sk_p, a.warmup, total, cs))
    elapsed = graph_s
    del g_sketch

    # ---- staggered windows (serving shape): every step updates N/W sequences -----------
    staggered = None
    if a.schedule == "staggered":
        N = cfg.batch
        taus = [torch.tensor([((ph + n) % W) + 1 for n in range(N)], dtype=torch.int32, device=dev)
                for ph in range(W)]
        ups = [torch.tensor([n for n in range(N) if ((ph + n) % W) + 1 == W], dtype=torch.int32,
                            device=dev) for ph in range(W)]
        fulls = [torch.full((len(u),), W, dtype=torch.int32, device=dev) for u in ups]
        d_ups = [ssm.Dims.make(cfg.rule, cfg.in_dtype, len(u), cfg.heads, cfg.d_k, cfg.d_v, W,
                               cfg.rank, a.sketch_dtype) for u in ups]
        tp, up, fp = [P(x) for x in taus], [P(x) for x in ups], [P(x) for x in fulls]

        def run_staggered(t_lo, t_hi, sp_, upd_events=None):
            for t in range(t_lo, t_hi):
                q, k, v, dc, b = ptrs[t]
                ph = t % W
                ssm.sketch_decode_step_varlen(d, N, None, tp[ph], sk_p, bp, q, kb, vb, db, bb, yp,
                                              k_t=k, v_t=v, decay_t=dc, beta_t=b, stream=sp_)
                if d_ups[ph].batch:
                    if upd_events is not None:
                        upd_events.append((torch.cuda.Event(enable_timing=True),
                                           torch.cuda.Event(enable_timing=True)))
                        upd_events[-1][0].record(stream)
                    ssm.window_update_refresh_varlen(d_ups[ph], N, up[ph], fp[ph], st_p, sk_p, bp,
                                                     kb, vb, db, bb, stream=sp_)
                    if upd_events is not None:
                        upd_events[-1][1].record(stream)

        run_staggered(0, a.warmup, sp)
        stg_ev = []
        eager_g = timed(lambda: run_staggered(a.warmup, total, sp, stg_ev))
        graph_g, g_stg = graph_timed(lambda cs: run_staggered(a.warmup, total, cs))
        del g_stg
        staggered = {"steps_per_s": a.steps / graph_g, "ms_per_step": graph_g * 1e3 / a.steps,
                     "eager_steps_per_s": a.steps / eager_g,
                     "update_per_step_ms": float(np.mean([s_.elapsed_time(e_) for s_, e_ in stg_ev])),
                     "sequences_updated_per_step": N / W}

    # ---- per-kernel time of the sketch read (events around each launch) ---------------
    def kernel_time(launch, reps):
        launch(0)  # untimed: the first launch of a kernel in a process also loads its code
        torch.cuda.synchronize()
        evs = []
        for i in range(reps):
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record(stream)
            launch(i)
            e_.record(stream)
            evs.append((s_, e_))
        torch.cuda.synchronize()
        return float(np.mean([s_.elapsed_time(e_) for s_, e_ in evs]))

    tau_mid = W // 2 + 1
    # bytes of one read at window position tau_mid, the token already buffered (no append):
    # q + tau_mid buffered tokens + y, plus the sketch (and read map) or the full state
    s_in = 2 if cfg.in_dtype == "bf16" else 4
    common = cfg.d_k * s_in + tau_mid * bm["tok"] + 4 * cfg.d_v
    sk_b = U * (bm["state_bytes_sketch"] + (4 * cfg.rank * cfg.d_k if ls else 0) + common)
    full_b = U * (bm["state_bytes_full"] + common)
    q0 = ptrs[0][0]
    sketch_ms = kernel_time(lambda i: sketch_step(sk_p, bp, q0, kb, vb, db, bb, tau_mid, yp,
                                                  stream=sp), 20)
    full_ms = kernel_time(lambda i: ssm.full_read_decode_step(d, st_p, q0, kb, vb, db, bb,
                                                              tau_mid, yp, stream=sp), 10)

    # ---- the exact full-read path on the same tokens (comparison) ----------------------
    full = None
    if not a.no_compare:
        state_f = S0_dev.clone()
        sf_p = P(state_f)
        run_full(sf_p, 0, a.warmup, sp)
        upd_f = []
        eager_f = timed(lambda: run_full(sf_p, a.warmup, total, sp, upd_f))
        graph_f, g_full = graph_timed(lambda cs: run_full(sf_p, a.warmup, total, cs))
        del g_full
        full = {"steps_per_s": a.steps / graph_f, "ms_per_step": graph_f * 1e3 / a.steps,
                "eager_steps_per_s": a.steps / eager_f,
                "update_no_refresh_ms": float(np.mean([s_.elapsed_time(e_) for s_, e_ in upd_f]))}
        del state_f

    # ---- the per-token recurrent decode (the standard baseline) on the same tokens -----
    per_token = None
    if not a.no_compare:
        state_r = S0_dev.clone()
        sr_p = P(state_r)

        def run_rec(state_p, t_lo, t_hi, sp_):
            for t in range(t_lo, t_hi):
                q, k, v, dc, b = ptrs[t]
                ssm.recurrent_decode_step(d, state_p, q, k, v, dc, b, yp, stream=sp_)

        run_rec(sr_p, 0, a.warmup, sp)
        eager_r = timed(lambda: run_rec(sr_p, a.warmup, total, sp))
        graph_r, g_rec = graph_timed(lambda cs: run_rec(sr_p, a.warmup, total, cs))
        del g_rec
        q0_, k0_, v0_, d0_, b0_ = ptrs[0]
        rec_ms = kernel_time(lambda i: ssm.recurrent_decode_step(d, sr_p, q0_, k0_, v0_, d0_, b0_,
                                                                 yp, stream=sp), 10)
        rec_bytes = U * (8 * cfg.d_k * cfg.d_v + bm["tok"] + cfg.d_k * (2 if cfg.in_dtype == "bf16" else 4)
                         + 4 * cfg.d_v)
        per_token = {"steps_per_s": a.steps / graph_r, "ms_per_step": graph_r * 1e3 / a.steps,
                     "eager_steps_per_s": a.steps / eager_r, "kernel_ms": rec_ms,
                     "kernel_gbs": rec_bytes / (rec_ms * 1e-3) / 1e9}
        del state_r

    # ---- approximation error of the sketch read vs the exact read (untimed) -----------
    st_a = S0_dev.clone()
    sk_a = torch.empty_like(sketch)
    if ls:
        rm_a = torch.empty((cfg.batch, cfg.heads, cfg.rank, cfg.d_k), device=dev)
        rmaps[sk_a.data_ptr()] = rm_a.data_ptr()
    update_refresh(st_a, sk_a, basis, None, None, None, None, 0, stream=stream)
    errs = []
    y_f = torch.empty_like(y)
    for t in range(2 * W):
        q, k, v, dc, b = inputs[t]
        tau = t % W + 1
        sketch_step(sk_a, basis, q, *bufs, tau, y, k_t=k, v_t=v, decay_t=dc, beta_t=b,
                               stream=stream)
        ssm.full_read_decode_step(d, st_a, q, *bufs, tau, y_f, stream=stream)
        num = (y - y_f).view(U, -1).norm(dim=1)
        den = y_f.view(U, -1).norm(dim=1)
        errs.append((num / den.clamp_min(1e-30)).cpu())
        if tau == W:
            update_refresh(st_a, sk_a, basis, *bufs, W, stream=stream)
    e = torch.cat(errs).double().numpy()
    approx = {"mean": float(e.mean()), "p50": float(np.median(e)), "p99": float(np.quantile(e, 0.99)),
              "max": float(e.max()), "steps": 2 * W}
    del st_a, sk_a

    # ---- attainable HBM rate: a plain device copy of 2 GiB (read + write) ---------------
    n_copy = (2 << 30) // 4
    src = torch.ones(n_copy, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = kernel_time(lambda i: dst.copy_(src), 5)
    copy_gbs = 2 * n_copy * 4 / (copy_ms * 1e-3) / 1e9
    del src, dst

    # ---- attainable HBM rate for the state's read + write: the library's in-place stream
    # probe over a buffer of the state's size, in the update's access order (shape 0) and in
    # flat 128 KB runs per workgroup (shape 1, the fastest plain shape measured) -----------
    n_tiles = (S0_dev.numel() * 4 // 65536) & ~1
    probe = torch.ones(n_tiles * 16384, device=dev)
    probe_gbs = []
    for shape in (0, 1):
        ms = kernel_time(lambda i: ssm.stream_probe(probe, n_tiles, shape, stream=sp), 10)
        probe_gbs.append(2 * n_tiles * 65536 / (ms * 1e-3) / 1e9)
    # and over a buffer whose read + write equals one sketch read's bytes: the ceiling of a
    # single short streaming launch of that size, launch and ramp included
    n_small = max(2, int(round(sk_b / 2 / 65536)) & ~1)
    small = probe[:n_small * 16384]
    small_ms = kernel_time(lambda i: ssm.stream_probe(small, n_small, 1, stream=sp), 20)
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
        st_c, sk_c = S0_dev.clone(), torch.empty_like(sketch)
        if ls:
            rm_c = torch.empty((cfg.batch, cfg.heads, cfg.rank, cfg.d_k), device=dev)
            rmaps[sk_c.data_ptr()] = rm_c.data_ptr()
        update_refresh(st_c, sk_c, basis, None, None, None, None, 0, stream=stream)

        def cold_time(launch, reps=5):
            evs = []
            launch()
            for i in range(reps):
                torch.sum(flush, dim=0, out=flush_sum)
                s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s_.record(stream)
                launch()
                e_.record(stream)
                evs.append((s_, e_))
            torch.cuda.synchronize()
            return float(np.mean([s_.elapsed_time(e_) for s_, e_ in evs]))

        stc_p, skc_p = P(st_c), P(sk_c)
        c_upd = cold_time(lambda: update_refresh(stc_p, skc_p, bp, kb, vb, db, bb, W, stream=sp))
        c_sk = cold_time(lambda: sketch_step(skc_p, bp, q0, kb, vb, db, bb, tau_mid, yp, stream=sp))
        c_full = cold_time(lambda: ssm.full_read_decode_step(d, stc_p, q0, kb, vb, db, bb,
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
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                key, sep, val = line.strip().partition(": ")
                if sep and key in ("config", "kernel_source_hash", "bytes_per_launch"):
                    tr[key] = val
        # counters taken on another kernel version do not describe this one
        # ... nor does a run on another workload (the counters are for the lockstep,
        # uniform-rank, fp32-sketch decode of that config)
        same_workload = (tr.get("config") == cfg.name and a.schedule == "lockstep"
                         and ranks is None and a.sketch_dtype == "f32" and not ls)
        if tr.get("kernel_source_hash") == kernel_source_hash() and same_workload:
            traffic = float(tr["bytes_per_launch"])

    # ---- CPU baseline: the oracle on a bounded sample --------------------------------
    cpu = None
    if not a.no_cpu_baseline:
        import oracle
        units = workloads.sample_units(cfg, min(a.cpu_units, U))
        Ts = min(a.cpu_steps, total)
        flat = lambda x, e: x.reshape((U,) + ((e,) if e else ()))[units]
        h = [steps_host[t] for t in range(Ts)]
        q = np.stack([workloads.widen(flat(s.q, cfg.d_k)) for s in h])
        k = np.stack([workloads.widen(flat(s.k, cfg.d_k)) for s in h])
        v = np.stack([workloads.widen(flat(s.v, cfg.d_v)) for s in h])
        dc = np.stack([flat(s.decay, cfg.d_k if cfg.per_channel_decay else 0) for s in h]).astype(np.float64)
        be = (np.stack([flat(s.beta, 0) for s in h]).astype(np.float64) if cfg.has_beta else None)
        S0s = S0.reshape(U, cfg.d_k, cfg.d_v)[units].astype(np.float64)
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

    value = a.steps / elapsed
    out = {
        "metric": metric_name(cfg),
        "value": value,
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": elapsed * 1e3 / a.steps,
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
                   "basis": "device fit" if a.fit_basis else "host"},
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
        "eager_steps_per_s": a.steps / eager_s,
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
        "input_gen_s": gen_s,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
