"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases (ragged unit counts, every rule, both input dtypes, all tile
shapes, a trailing partial window) are compared on every unit; the workload
sizes are compared on a sample of units (always the first and the last) at
every step and after every window, in the same launch configuration the
benchmark times.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import workloads
import sketched_recurrent_state_amd as ssm
from sketched_recurrent_state_amd.decoder import WindowedDecoder
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


BASE = {"mamba2": workloads.C2, "gdn": workloads.C3, "kda": workloads.C4}


def small(rule, in_dtype="bf16", d_k=128, d_v=128, W=8, r=8, N=3, Hh=5, T=None):
    cfg = BASE[rule].with_(name=f"small_{rule}_{in_dtype}_{d_k}x{d_v}_w{W}_r{r}",
                           in_dtype=in_dtype, batch=N, heads=Hh, d_k=d_k, d_v=d_v,
                           window=W, rank=r)
    return cfg.with_(steps=T if T is not None else 2 * W + 3)


SMALL = [
    small("mamba2"), small("gdn"), small("kda"),
    small("mamba2", d_k=128, d_v=64), small("gdn", d_k=64, d_v=32, W=5, r=3),
    small("kda", d_k=32, d_v=64, W=3, r=32), small("gdn", d_k=16, d_v=32, W=16, r=1),
    small("kda", d_k=16, d_v=128, W=1, r=16), small("mamba2", d_k=32, d_v=128, W=2, r=9),
    small("gdn", "f32", d_k=64, d_v=64, W=4, r=16), small("kda", "f32", d_k=128, d_v=32, W=6, r=8),
    small("mamba2", "f32", d_k=16, d_v=64, W=3, r=16),
    small("gdn", N=7, Hh=9, W=8, r=8),   # 63 units: a ragged last wave of the sketch read
    # 32 x 32 (one wave per unit): every rule, r = d_k = 32 included (a full basis)
    small("gdn", d_k=32, d_v=32, W=7, r=5), small("mamba2", d_k=32, d_v=32, W=2, r=1),
    small("kda", "f32", d_k=32, d_v=32, W=12, r=32, T=27),
    # the largest supported shapes: LDS and registers at their maximum
    small("kda", "f32", d_k=128, d_v=128, W=16, r=32, N=2, Hh=3, T=35),
    small("gdn", "bf16", d_k=128, d_v=128, W=16, r=32, N=2, Hh=3, T=33),
]


# More shapes at the model sizes (d_k, d_v in {64, 128}): odd windows, W = 1 and 16, ranks
# from 1 to 30, both input types.
MODEL_SHAPES = [
    small("gdn", d_k=64, d_v=128, W=6, r=5),
    small("mamba2", d_k=64, d_v=64, W=7, r=12),
    small("gdn", "f32", d_k=128, d_v=64, W=3, r=2),
    small("mamba2", d_k=128, d_v=128, W=16, r=16, T=37),
    small("gdn", d_k=64, d_v=64, W=1, r=1, T=5),
    # a basis of 1,536 floats: a second 1,024-float LDS chunk, half of it a clamped tail
    small("kda", d_k=64, d_v=128, W=8, r=24, T=19),
    small("gdn", "f32", d_k=128, d_v=128, W=13, r=30, N=2, Hh=3, T=29),
]
SMALL += MODEL_SHAPES

# d_v = 16: one wave per unit with 4 column groups and 16 row groups (the d_k reductions
# take lane bit 2 as well); every rule, both input types, W from 1 to 16, ranks 1 to 32.
DV16 = [
    small("gdn", d_k=128, d_v=16, W=8, r=8),
    small("kda", d_k=64, d_v=16, W=5, r=16),
    small("mamba2", "f32", d_k=16, d_v=16, W=3, r=4),
    small("gdn", "f32", d_k=32, d_v=16, W=16, r=32, T=35),
    small("kda", d_k=128, d_v=16, W=1, r=1, T=5),
    small("mamba2", d_k=128, d_v=16, W=4, r=12, N=7, Hh=9),
]
SMALL += DV16

# Windows of 9 to 16 tokens for Mamba-2 and GDN (the windows where the update's FMAs, not
# HBM, come closest to setting its pace): both rules, both input types, d_k and d_v from
# 32 to 128 (one to four waves per unit), ranks 1 to 16, a last window cut short.
CHUNK = [
    small("gdn", W=16, r=8, N=3, Hh=4, T=35),
    small("mamba2", d_k=128, d_v=64, W=12, r=5, T=27),
    small("gdn", "f32", d_k=64, d_v=32, W=9, r=16, T=21),
    small("gdn", d_k=32, d_v=128, W=11, r=13, T=25),
    small("mamba2", "f32", d_k=64, d_v=128, W=16, r=1, T=35),
    small("gdn", d_k=128, d_v=32, W=14, r=3, N=5, Hh=3, T=30),
]
SMALL += CHUNK


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_all_units(cfg):
    H.note(f"case {cfg.name}")
    units = np.arange(cfg.units)
    inp = H.Inputs(cfg, units, cfg.steps)
    got = H.run_gpu(cfg, inp)
    ref = H.run_oracle(cfg, inp)
    H.compare(cfg, got, ref)


def test_c1_tiny_mamba2_fp32():
    cfg = workloads.C1
    H.note("case c1")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    H.compare(cfg, H.run_gpu(cfg, inp), H.run_oracle(cfg, inp))


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_workload_sampled_units(name):
    cfg = workloads.get(name)
    H.note(f"case {name} (sampled units)")
    units = workloads.sample_units(cfg, 40)
    inp = H.Inputs(cfg, units, cfg.steps)
    got = H.run_gpu(cfg, inp)
    ref = H.run_oracle(cfg, inp)
    H.compare(cfg, got, ref)


@pytest.fixture(scope="module")
def c5_inputs():
    cfg = workloads.c5(8, 8)
    return H.Inputs(cfg, workloads.sample_units(cfg, 16), cfg.steps)


@pytest.mark.parametrize("r,W", [(r, W) for r in workloads.C5_RANKS for W in workloads.C5_WINDOWS])
def test_c5_sweep_sampled_units(c5_inputs, r, W):
    cfg = workloads.c5(r, W)
    H.note(f"case {cfg.name} (sampled units)")
    inp = c5_inputs
    # the sweep shares one token stream; only the basis follows the rank
    B = workloads.basis(cfg)
    inp.basis = torch.from_numpy(B).cuda()
    inp.host_basis = B[inp.units % cfg.heads].astype(np.float64)
    got = H.run_gpu(cfg, inp, check_state_frozen=(r == 8 and W == 8))
    H.compare(cfg, got, H.run_oracle(cfg, inp))


def test_fused_append_equals_separate_append():
    cfg = small("kda", W=4, r=8)
    H.note("case fused-vs-separate append")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    a = H.run_gpu(cfg, inp, fused=True)
    b = H.run_gpu(cfg, inp, fused=False)
    for key in ("y_sketch", "y_full", "S", "Sk"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("rule", ["mamba2", "gdn", "kda"])
def test_full_read_fused_append(rule):
    """The exact full-read path on its own, with the current token appended inside the
    full-read kernel (as the bench's comparison path runs it): outputs and window-start
    states against the oracle's exact read, and the window buffer after every step, the
    outputs and the states bit for bit equal to a run with separate append launches."""
    cfg = small(rule, W=4, T=11)   # two full windows and a partial one
    H.note(f"case full read with fused append {rule}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    a = H.run_gpu_full(cfg, inp, fused=True, keep_buffers=True)
    b = H.run_gpu_full(cfg, inp, fused=False, keep_buffers=True)
    for t, (ba, bb) in enumerate(zip(a["bufs"], b["bufs"])):
        for name, x, z in zip(("k_buf", "v_buf", "decay_buf", "beta_buf"), ba, bb):
            assert (x is None and z is None) or torch.equal(x, z), f"step {t}: {name} differs"
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["S"], b["S"])
    ref = H.run_oracle(cfg, inp)
    e = H.rel_rows(a["y"], ref["y_exact"])
    scale = np.maximum(np.max(np.abs(ref["y_exact"]), axis=-1, keepdims=True), 1e-30)
    el = float(np.max(np.abs(a["y"] - ref["y_exact"]) / scale))
    H.note(f"full read {rule}: y {e.max():.2e} (element {el:.2e})")
    assert e.max() <= H.Y_TOL and el <= H.Y_TOL
    H.assert_mats(a["S"], ref["S_win"][:a["S"].shape[0]], H.S_TOL, "state")


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_full_read_workload_sampled(name):
    """The exact full-read path at a workload's size (C3: the GDN layer, N=256, H=32, 128x128,
    W=8), with the fused append, in the launch configuration the bench's comparison leg times;
    40 sampled units, every step and window."""
    cfg = workloads.get(name)
    H.note(f"case full read {name} (sampled units)")
    inp = H.Inputs(cfg, workloads.sample_units(cfg, 40), cfg.steps)
    got = H.run_gpu_full(cfg, inp, fused=True)
    ref = H.run_oracle(cfg, inp)
    e = H.rel_rows(got["y"], ref["y_exact"])
    H.note(f"full read {name}: y {e.max():.2e}")
    assert e.max() <= H.Y_TOL
    H.assert_mats(got["S"], ref["S_win"], H.S_TOL, "state")


def test_two_runs_are_bitwise_equal():
    cfg = small("gdn", N=16, Hh=8)
    H.note("case determinism")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    a = H.run_gpu(cfg, inp)
    b = H.run_gpu(cfg, inp)
    for key in ("y_sketch", "y_full", "S", "Sk"):
        assert np.array_equal(a[key], b[key]), key
    assert torch.equal(a["final_state"], b["final_state"])


@pytest.mark.parametrize("rule,W,n", [("mamba2", 8, 5), ("gdn", 8, 5), ("kda", 8, 5),
                                      ("mamba2", 16, 11), ("gdn", 16, 11)])
def test_partial_window_flush(rule, W, n):
    """n < W buffered tokens written early: the state equals the recurrence after n tokens."""
    cfg = small(rule, W=W, T=n)
    H.note(f"case partial flush {rule} W={W} n={n}")
    inp = H.Inputs(cfg, np.arange(cfg.units), n)
    d = H.dims_of(cfg)
    state = inp.S0.clone()
    dec = WindowedDecoder(d, state, inp.basis, read="sketch")
    dec.refresh()
    ys = []
    for t in range(n):
        ys.append(dec.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t]).clone())
    dec.flush()
    torch.cuda.synchronize()
    ref = H.run_oracle(cfg.with_(window=n), inp)   # one window of n tokens
    U = cfg.units
    got_S = state.view(1, U, cfg.d_k, cfg.d_v).cpu().double().numpy()
    H.assert_mats(got_S, ref["S_win"][1:2], H.S_TOL, "state after the flush")
    got_Sk = dec.sketch.view(1, U, cfg.rank, cfg.d_v).cpu().double().numpy()
    H.assert_mats(got_Sk, ref["Sk"][1:2], H.S_TOL, "sketch after the flush")
    got_y = torch.stack(ys).view(n, U, cfg.d_v).cpu().double().numpy()
    assert H.rel_rows(got_y, ref["y_sketch"]).max() <= H.Y_TOL


def test_nan_stays_in_its_unit():
    """A NaN key in one unit poisons that unit only."""
    cfg = small("gdn", N=4, Hh=4, W=4, T=8)
    H.note("case unit isolation")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    clean = H.run_gpu(cfg, inp, check_state_frozen=False)
    bad_unit = 5
    k2 = inp.k[2].clone()
    k2.view(cfg.units, -1)[bad_unit, 3] = float("nan")
    inp.k[2] = k2
    dirty = H.run_gpu(cfg, inp, check_state_frozen=False)
    others = [u for u in range(cfg.units) if u != bad_unit]
    for key in ("y_sketch", "y_full"):
        assert np.array_equal(clean[key][:, others], dirty[key][:, others]), key
        assert np.isnan(dirty[key][2:, bad_unit]).all(), key
    assert np.array_equal(clean["S"][:, others], dirty["S"][:, others])


def test_outputs_stay_inside_their_arrays():
    """Guard bands around y, the sketch and the state are never written."""
    cfg = small("kda", N=2, Hh=3, W=4, r=8, T=4)
    H.note("case guard bands")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    d = H.dims_of(cfg)
    U = cfg.units
    pad = 1024
    sentinel = 12345.0

    def guarded(n):
        buf = torch.full((n + 2 * pad,), sentinel, device="cuda")
        return buf, buf[pad:pad + n]

    sbuf, S = guarded(U * cfg.d_k * cfg.d_v)
    S.copy_(inp.S0.view(-1))
    kbuf, skv = guarded(U * cfg.rank * cfg.d_v)
    ybuf, yv = guarded(U * cfg.d_v)
    y2buf, y2v = guarded(U * cfg.d_v)
    dec = WindowedDecoder(d, S.view(cfg.batch, cfg.heads, cfg.d_k, cfg.d_v), inp.basis, read="both")
    dec.sketch = skv.view(cfg.batch, cfg.heads, cfg.rank, cfg.d_v)
    dec.refresh()
    for t in range(cfg.steps):
        dec.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t],
                 y=yv.view(cfg.batch, cfg.heads, cfg.d_v), y_full=y2v.view(cfg.batch, cfg.heads, cfg.d_v))
    torch.cuda.synchronize()
    for buf in (sbuf, kbuf, ybuf, y2buf):
        assert (buf[:pad] == sentinel).all() and (buf[-pad:] == sentinel).all()


def test_empty_batch_on_device():
    d = ssm.Dims.make("gdn", "bf16", 0, 4, 128, 128, 8, 8)
    z = torch.empty(0, device="cuda")
    ssm.window_update_refresh(d, z, z, torch.zeros(4 * 8 * 128, device="cuda"), None, None, None,
                              None, 0)
    torch.cuda.synchronize()


RECURRENT = [small("mamba2"), small("gdn"), small("kda"), small("gdn", "f32", d_k=64, d_v=32),
             small("kda", d_k=16, d_v=128), small("mamba2", "f32", d_k=32, d_v=64),
             small("kda", "f32", d_k=128, d_v=32),   # d_k staged in two passes of 64 threads
             small("gdn", d_k=128, d_v=16), small("kda", "f32", d_k=32, d_v=16)]


@pytest.mark.parametrize("cfg", RECURRENT, ids=lambda c: c.name)
def test_recurrent_step_small(cfg):
    """The per-token baseline: exact read of the state after each token, state written each step."""
    H.note(f"case recurrent {cfg.name}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    H.compare_recurrent(cfg, H.run_gpu_recurrent(cfg, inp), inp)


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_recurrent_step_workload_sampled(name):
    cfg = workloads.get(name).with_(steps=24)
    H.note(f"case recurrent {name} (sampled units, 24 steps)")
    inp = H.Inputs(cfg, workloads.sample_units(cfg, 24), cfg.steps)
    H.compare_recurrent(cfg, H.run_gpu_recurrent(cfg, inp), inp)


def _ranked_case(cfg, ranks, steps=None):
    """Per-head ranks: the GPU's ranked entry points against the oracle run per rank group."""
    import oracle
    steps = steps or cfg.steps
    units = np.arange(cfg.units) if cfg.units <= 64 else workloads.sample_units(cfg, 32)
    inp = H.Inputs(cfg, units, steps)
    B = workloads.basis_ranked(cfg, ranks)
    off = np.concatenate([[0], np.cumsum(ranks)])
    d = H.dims_of(cfg.with_(rank=max(ranks)))
    U, W, R = cfg.units, cfg.window, int(off[-1])
    state = inp.S0.clone()
    dec = WindowedDecoder(d, state, torch.from_numpy(B).cuda(), read="both", ranks=ranks)
    dec.refresh()
    ys, sks = [], [dec.sketch.clone()]
    for t in range(steps):
        y, _ = dec.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t])
        ys.append(y.view(U, -1)[torch.as_tensor(units, device="cuda")].cpu().double().numpy())
        if (t + 1) % W == 0:
            sks.append(dec.sketch.clone())
    torch.cuda.synchronize()
    ys = np.stack(ys)
    heads = units % cfg.heads
    h = inp.host
    worst = 0.0
    for r in sorted(set(ranks)):
        sel = np.nonzero(np.array([ranks[x] == r for x in heads]))[0]
        if sel.size == 0:
            continue
        Bu = np.stack([B[off[heads[i]]:off[heads[i]] + r] for i in sel]).astype(np.float64)
        ref = oracle.run(cfg.rule, inp.host_S0[sel], Bu, h["q"][:, sel], h["k"][:, sel],
                         h["v"][:, sel], h["decay"][:, sel],
                         None if h["beta"] is None else h["beta"][:, sel], W)
        e = H.rel_rows(ys[:, sel], ref["y_sketch"])
        worst = max(worst, float(e.max()))
        assert e.max() <= H.Y_TOL, f"rank {r}: sketch read max rel err {e.max():.3e}"
        for w, sk in enumerate(sks):
            got = np.stack([sk.view(cfg.batch, R, cfg.d_v)[units[i] // cfg.heads,
                                                          off[heads[i]]:off[heads[i]] + r]
                            .cpu().double().numpy() for i in sel])
            H.assert_mats(got[None], ref["Sk"][w][None], H.S_TOL, f"rank {r}: sketch after window {w}")
    H.note(f"ranked {cfg.name} ranks={sorted(set(ranks))}: max sketch-read err {worst:.2e}")


@pytest.mark.parametrize("rule", ["mamba2", "gdn"])
def test_per_head_ranks_window_16(rule):
    """Per-head ranks up to 16 with a 16-token window."""
    cfg = small(rule, N=3, Hh=5, W=16, T=35)
    H.note(f"case per-head ranks, 16-token window, {rule}")
    _ranked_case(cfg, [1, 8, 3, 16, 12])


@pytest.mark.parametrize("rule", ["mamba2", "gdn", "kda"])
def test_per_head_ranks_small(rule):
    cfg = small(rule, N=3, Hh=5, W=4, T=11)
    H.note(f"case per-head ranks {rule}")
    _ranked_case(cfg, [1, 8, 3, 16, 32])


@pytest.mark.parametrize("rule", ["mamba2", "gdn", "kda"])
def test_per_head_ranks_above_eight(rule):
    """Odd and even ranks above the eight sketch rows fetched with the step's other loads
    (9, 16, 17, 25: further fetches of one to eight live rows), beside ranks of 8 and below in
    the same launch, over 5 rows (a ragged workgroup)."""
    cfg = small(rule, N=5, Hh=6, W=8, T=19)
    H.note(f"case per-head ranks above 8, {rule}")
    _ranked_case(cfg, [9, 17, 2, 25, 8, 16])


@pytest.mark.parametrize("rule", ["mamba2", "gdn", "kda"])
def test_per_head_ranks_bf16_sketch(rule):
    """Per-head ranks with the sketch stored in bf16: for every rank group, both reads, the
    state and the stored sketch against the oracle's bf16 mode, with the oracle-only rounding
    windows of the uniform-rank bf16 tests."""
    import oracle
    cfg = small(rule, N=3, Hh=5, W=4, T=11)
    ranks = [1, 8, 3, 16, 12]
    H.note(f"case per-head ranks, bf16 sketch, {rule}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    B = workloads.basis_ranked(cfg, ranks)
    off = np.concatenate([[0], np.cumsum(ranks)])
    d = H.dims_of(cfg.with_(rank=max(ranks)), "bf16")
    U, W, R = cfg.units, cfg.window, int(off[-1])
    state = inp.S0.clone()
    dec = WindowedDecoder(d, state, torch.from_numpy(B).cuda(), read="both", ranks=ranks)
    dec.refresh()
    ys, yf = [], []
    S_snap = [state.view(U, cfg.d_k, cfg.d_v).cpu().double().numpy()]
    Sk_snap = [dec.sketch.view(cfg.batch, R, cfg.d_v).float().cpu().double().numpy()]
    for t in range(cfg.steps):
        y, y2 = dec.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t])
        ys.append(y.view(U, -1).cpu().double().numpy())
        yf.append(y2.view(U, -1).cpu().double().numpy())
        if (t + 1) % W == 0:
            S_snap.append(state.view(U, cfg.d_k, cfg.d_v).cpu().double().numpy())
            Sk_snap.append(dec.sketch.view(cfg.batch, R, cfg.d_v).float().cpu().double().numpy())
    torch.cuda.synchronize()
    ys, yf, S_snap = np.stack(ys), np.stack(yf), np.stack(S_snap)
    heads = np.arange(U) % cfg.heads
    h = inp.host
    for r in sorted(set(ranks)):
        sel = np.nonzero(np.array([ranks[x] == r for x in heads]))[0]
        Bu = np.stack([B[off[heads[i]]:off[heads[i]] + r] for i in sel]).astype(np.float64)
        args = (cfg.rule, inp.host_S0[sel], Bu, h["q"][:, sel], h["k"][:, sel], h["v"][:, sel],
                h["decay"][:, sel], None if h["beta"] is None else h["beta"][:, sel], W)
        ref = oracle.run(*args, sketch_bf16=True, want_ls=True)
        ref_exact = oracle.run(*args)
        sk = np.stack([np.stack([Sk_snap[w][i // cfg.heads, off[heads[i]]:off[heads[i]] + r]
                                 for i in sel]) for w in range(len(Sk_snap))])
        got = dict(y_sketch=ys[:, sel], y_full=yf[:, sel], S=S_snap[:, sel], Sk=sk)
        H.compare(cfg.with_(rank=r), got, ref, sketch_bf16=True, host_basis=Bu,
                  ref_exact=ref_exact)


@pytest.mark.parametrize("rule", ["mamba2", "gdn", "kda"])
def test_per_head_ranks_f32_inputs(rule):
    """Per-head ranks with fp32 q, k, v: ranks on both sides of the eight fetched ahead, an
    odd window."""
    cfg = small(rule, "f32", d_k=64, d_v=64, N=3, Hh=5, W=6, T=13)
    H.note(f"case per-head ranks, fp32 inputs, {rule}")
    _ranked_case(cfg, [4, 9, 2, 17, 8])


def test_per_head_ranks_d_v_16():
    cfg = small("gdn", d_k=64, d_v=16, N=3, Hh=5, W=4, T=11)
    H.note("case per-head ranks d_v=16")
    _ranked_case(cfg, [1, 8, 3, 16, 32])


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_per_head_ranks_average_8_workload(name):
    """A workload at full size with a mean-8 rank pattern (2, 4, 8, 18 cycled over heads)."""
    cfg = workloads.get(name).with_(steps=24)
    H.note(f"case per-head ranks {name} (sampled units)")
    _ranked_case(cfg, workloads.average_rank_8(cfg.heads))


@pytest.mark.parametrize("rule", ["mamba2", "gdn", "kda"])
def test_continuous_batching_varlen(rule):
    """Sequences join at different steps into permuted pool slots, each at its own window
    position; a padding row (tau = 0) is skipped and its output left untouched; update calls
    skip rows whose window is not full (n_tokens = -1). Every sequence is checked against its
    own oracle run over its local steps."""
    import oracle
    W, T = 4, 14
    joins = [0, 1, 2, 3, 5, 6]
    slots = [5, 0, 7, 2, 3, 6]
    P = 8                                      # pool size
    cfg = small(rule, d_k=64, d_v=64, W=W, r=8, N=len(joins), Hh=3, T=T)
    H.note(f"case continuous batching {rule}")
    Hh, dk, dv = cfg.heads, cfg.d_k, cfg.d_v
    S0 = np.concatenate([workloads.initial_state(cfg, [n]) for n in range(len(joins))])
    B = workloads.basis(cfg)
    steps = [workloads.step_inputs(cfg, j) for j in range(T)]   # local step j, row n = sequence n
    d_pool = H.dims_of(cfg.with_(batch=P))
    dev = "cuda"
    tin = torch.bfloat16

    def td(x):
        return None if x is None else H._to_dev(np.ascontiguousarray(x), dev)

    state = torch.zeros((P, Hh, dk, dv), device=dev)
    sketch = torch.zeros((P, Hh, cfg.rank, dv), device=dev)
    kb = torch.zeros((P, Hh, W, dk), device=dev, dtype=tin)
    vb = torch.zeros((P, Hh, W, dv), device=dev, dtype=tin)
    dshape = (P, Hh, W, dk) if rule == "kda" else (P, Hh, W)
    db = torch.zeros(dshape, device=dev)
    bb = torch.zeros((P, Hh, W), device=dev) if rule != "mamba2" else None
    basis = td(B)
    got_y = {n: [] for n in range(len(joins))}
    sentinel = 777.0
    for t in range(T):
        joining = [n for n in range(len(joins)) if joins[n] == t]
        for n in joining:
            state[slots[n]] = torch.from_numpy(S0[n]).to(dev)
        if joining:   # refresh-only pass for the sequences that just joined
            dj = cfg.with_(batch=len(joining))
            ssm.window_update_refresh_varlen(
                H.dims_of(dj), P, td(np.array([slots[n] for n in joining], np.int32)),
                td(np.zeros(len(joining), np.int32)), state, sketch, basis, kb, vb, db, bb)
        active = [n for n in range(len(joins)) if joins[n] <= t][::-1]   # reversed row order
        rows = active + [None]                                          # + one padding row
        tau = [((t - joins[n]) % W) + 1 if n is not None else 0 for n in rows]
        slot_rows = [slots[n] if n is not None else 1 for n in rows]
        pick = lambda x, n: x[n] if n is not None else np.zeros_like(x[0])
        loc = lambda n: t - joins[n] if n is not None else 0
        q = np.stack([pick(steps[loc(n)].q, n) for n in rows])
        k = np.stack([pick(steps[loc(n)].k, n) for n in rows])
        v = np.stack([pick(steps[loc(n)].v, n) for n in rows])
        dc = np.stack([pick(steps[loc(n)].decay, n) for n in rows])
        bt = (np.stack([pick(steps[loc(n)].beta, n) for n in rows]) if rule != "mamba2" else None)
        dr = H.dims_of(cfg.with_(batch=len(rows)))
        y = torch.full((len(rows), Hh, dv), sentinel, device=dev)
        ssm.sketch_decode_step_varlen(dr, P, td(np.array(slot_rows, np.int32)),
                                      td(np.array(tau, np.int32)), sketch, basis, td(q), kb, vb,
                                      db, bb, y, k_t=td(k), v_t=td(v), decay_t=td(dc),
                                      beta_t=td(bt))
        yc = y.cpu().double().numpy()
        assert (yc[-1] == sentinel).all(), "padding row was written"
        for i, n in enumerate(active):
            got_y[n].append(yc[i])
        # windows that just filled: update them; the others are skipped with n_tokens = -1
        ntok = np.array([W if tau[i] == W else -1 for i in range(len(active))], np.int32)
        ssm.window_update_refresh_varlen(H.dims_of(cfg.with_(batch=len(active))), P,
                                         td(np.array(slot_rows[:-1], np.int32)), td(ntok),
                                         state, sketch, basis, kb, vb, db, bb)
    torch.cuda.synchronize()
    for n in range(len(joins)):
        Tn = T - joins[n]
        wid = lambda x, e: x.reshape((cfg.batch, Hh) + ((e,) if e else ()))[n]
        hq = np.stack([workloads.widen(wid(steps[j].q, dk)) for j in range(Tn)])
        hk = np.stack([workloads.widen(wid(steps[j].k, dk)) for j in range(Tn)])
        hv = np.stack([workloads.widen(wid(steps[j].v, dv)) for j in range(Tn)])
        hd = np.stack([wid(steps[j].decay, dk if rule == "kda" else 0) for j in range(Tn)]).astype(np.float64)
        hb = (np.stack([wid(steps[j].beta, 0) for j in range(Tn)]).astype(np.float64)
              if rule != "mamba2" else None)
        ref = oracle.run(rule, S0[n].astype(np.float64), B.astype(np.float64), hq, hk, hv, hd, hb, W)
        e = H.rel_rows(np.stack(got_y[n]), ref["y_sketch"])
        assert e.max() <= H.Y_TOL, f"sequence {n}: sketch read {e.max():.3e}"
        nw = Tn // W
        gS = state[slots[n]].cpu().double().numpy()
        H.assert_mats(gS[None, None], ref["S_win"][nw][None, None], H.S_TOL, f"sequence {n}: state")
        gK = sketch[slots[n]].cpu().double().numpy()
        H.assert_mats(gK[None, None], ref["Sk"][nw][None, None], H.S_TOL, f"sequence {n}: sketch")
    # slot 4 and 1 were never assigned to a sequence: untouched
    assert torch.count_nonzero(state[4]) == 0 and torch.count_nonzero(state[1]) == 0


def test_checkpoint_mid_window_and_resume():
    """A mid-window checkpoint (state, sketch, window buffer) restored into fresh memory
    continues bitwise identically to the uninterrupted run."""
    cfg = small("gdn", W=8, T=20)
    H.note("case checkpoint / resume")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    d = H.dims_of(cfg)
    a = WindowedDecoder(d, inp.S0.clone(), inp.basis, read="sketch")
    a.refresh()
    ya = []
    cut = 11   # three tokens into the second window
    b = None
    for t in range(cfg.steps):
        if t == cut:
            b = WindowedDecoder(d, a.state.clone(), inp.basis, read="sketch")
            for name in ("sketch", "k_buf", "v_buf", "decay_buf", "beta_buf"):
                getattr(b, name).copy_(getattr(a, name))
            b.tau = a.tau
            yb = []
        ya.append(a.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t]).clone())
        if b is not None:
            yb.append(b.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t]).clone())
    torch.cuda.synchronize()
    for i, y in enumerate(yb):
        assert torch.equal(y, ya[cut + i]), f"step {cut + i}"
    assert torch.equal(a.state, b.state) and torch.equal(a.sketch, b.sketch)


@pytest.mark.parametrize("rule,W", [("mamba2", 4), ("gdn", 4), ("kda", 4), ("mamba2", 12),
                                    ("gdn", 12)])
def test_extreme_gates(rule, W):
    """Exact zero gates (they clear everything before them), gates of 1, beta of 0 and 1,
    and a large-magnitude state: the suffix-product update and the walk match the oracle,
    at W = 4 and W = 12."""
    cfg = small(rule, N=3, Hh=4, W=W, T=3 * W)
    H.note(f"case extreme gates {rule} W={W}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    U = cfg.units
    rng = np.random.default_rng(7)
    for t in range(cfg.steps):
        dec = inp.decay[t].clone().view(U, -1)
        pick = rng.integers(0, 4, size=U)
        dec[torch.as_tensor(pick == 0, device="cuda")] = 0.0
        dec[torch.as_tensor(pick == 1, device="cuda")] = 1.0
        inp.decay[t] = dec.view_as(inp.decay[t])
        hd = inp.host["decay"][t].reshape(U, -1)
        hd[pick == 0] = 0.0
        hd[pick == 1] = 1.0
        if inp.beta[t] is not None:
            bsel = rng.integers(0, 3, size=U)
            b = inp.beta[t].clone().view(U)
            b[torch.as_tensor(bsel == 0, device="cuda")] = 0.0
            b[torch.as_tensor(bsel == 1, device="cuda")] = 1.0
            inp.beta[t] = b.view_as(inp.beta[t])
            hb = inp.host["beta"][t]
            hb[bsel == 0] = 0.0
            hb[bsel == 1] = 1.0
    inp.S0 = inp.S0 * 1e3
    inp.host_S0 = inp.host_S0 * 1e3
    H.compare(cfg, H.run_gpu(cfg, inp), H.run_oracle(cfg, inp))


# bf16 sketch storage: the sketch is rounded to bf16 when the refresh stores it;
# the oracle rounds its sketch the same way. Rules, input types, odd shapes,
# per-head ranks do not change the path, so one of each shape family is enough.
BF16_SKETCH = [
    small("gdn"), small("kda", W=4, r=8), small("mamba2", d_k=128, d_v=64),
    small("gdn", "f32", d_k=64, d_v=32, W=5, r=3), small("kda", d_k=16, d_v=128, W=1, r=16),
    small("gdn", "bf16", d_k=128, d_v=128, W=16, r=32, N=2, Hh=3, T=33),
    small("kda", d_k=64, d_v=16, W=4, r=8),
    small("gdn", W=16, r=8, N=2, Hh=3, T=33), small("mamba2", d_k=64, d_v=64, W=10, r=12),
]


@pytest.mark.parametrize("cfg", BF16_SKETCH, ids=lambda c: c.name)
def test_bf16_sketch(cfg):
    H.note(f"case bf16 sketch {cfg.name}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    got = H.run_gpu(cfg, inp, sketch_dtype="bf16")
    ref = H.run_oracle(cfg, inp, sketch_bf16=True, want_ls=True)  # want_ls: q~ for the slack
    ref_exact = H.run_oracle(cfg, inp)                             # the unrounded sketch
    H.compare(cfg, got, ref, sketch_bf16=True, host_basis=inp.host_basis, ref_exact=ref_exact)
    assert got["sketch"].dtype == torch.bfloat16


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_bf16_sketch_workload_sampled(name):
    """A workload at full size with the bf16 sketch, as bench.py times it; 40 sampled units,
    every step and window."""
    cfg = workloads.get(name)
    H.note(f"case bf16 sketch {name} (sampled units)")
    inp = H.Inputs(cfg, workloads.sample_units(cfg, 40), cfg.steps)
    got = H.run_gpu(cfg, inp, sketch_dtype="bf16")
    ref = H.run_oracle(cfg, inp, sketch_bf16=True, want_ls=True)  # want_ls: q~ for the slack
    ref_exact = H.run_oracle(cfg, inp)                             # the unrounded sketch
    H.compare(cfg, got, ref, sketch_bf16=True, host_basis=inp.host_basis, ref_exact=ref_exact)


# Least-squares coefficients: the read is the projection of the exact window-start
# read on the span of the sketch rows; the refresh stores orthonormal sketch rows Q
# and the per-unit read map Y = Q S^T.
LS_CASES = [
    small("gdn"), small("mamba2", d_k=128, d_v=64), small("kda", W=4, r=8),
    small("gdn", "f32", d_k=64, d_v=32, W=5, r=3),
    small("kda", d_k=16, d_v=128, W=1, r=16),   # r = d_k: the read is exact
    # d_v = 16: 4 lanes per row group; factorisation in registers (r = 8) and in LDS (r = 12),
    # and r = 24 > d_v, where the rows past the 16th are dependent and dropped (the read is
    # then the exact window-start read)
    small("gdn", d_k=128, d_v=16, W=8, r=8), small("kda", d_k=64, d_v=16, W=5, r=12),
    small("mamba2", "f32", d_k=32, d_v=16, W=3, r=24),
    small("gdn", "bf16", d_k=128, d_v=128, W=16, r=32, N=2, Hh=3, T=33),
]


def check_least_squares(cfg, got, ref):
    """Least-squares parity on the units the run sampled."""
    nw, n = got["S"].shape[0], got["S"].shape[1]
    e_y = H.rel_rows(got["y_sketch"], ref["y_ls"])
    e_x = H.rel_rows(got["y_full"], ref["y_exact"])
    e_S = H.assert_mats(got["S"], ref["S_win"][:nw], H.S_TOL, "least-squares state")
    # the stored rows are orthonormal, or exactly zero where the factorisation dropped a
    # dependent row, and span the oracle's sketch rows
    Q = got["Sk"]
    gram = np.einsum("wuij,wukj->wuik", Q, Q)
    kept = np.einsum("wuii->wui", gram) > 0.5
    assert np.all(Q[~kept] == 0.0), "a dropped sketch row is not stored as zero"
    target = np.where(kept[..., :, None] & kept[..., None, :], np.eye(cfg.rank), 0.0)
    e_orth = np.abs(gram - target).max()
    Sk = ref["Sk"][:nw]
    resid = Sk - np.einsum("wuij,wujk->wuik", np.einsum("wuij,wukj->wuik", Sk, Q), Q)
    e_span = float((np.linalg.norm(resid.reshape(nw, n, -1), axis=-1)
                    / np.linalg.norm(Sk.reshape(nw, n, -1), axis=-1)).max())
    approx_ls = H.rel_rows(ref["y_ls"], ref["y_exact"]).mean()
    approx_pr = H.rel_rows(ref["y_sketch"], ref["y_exact"]).mean()
    H.note(f"least squares {cfg.name}: y {e_y.max():.2e} exact {e_x.max():.2e} S {e_S:.2e} "
           f"orth {e_orth:.2e} span {e_span:.2e} approx err {approx_ls:.3f} (projection {approx_pr:.3f})")
    assert e_y.max() <= H.Y_TOL, f"least-squares read: {e_y.max():.3e}"
    assert e_x.max() <= H.Y_TOL
    assert e_orth <= 1e-5, f"sketch rows not orthonormal: {e_orth:.2e}"
    assert e_span <= H.S_TOL, f"sketch rows do not span the sketch: {e_span:.2e}"
    if cfg.rank == cfg.d_k:
        assert H.rel_rows(got["y_sketch"], ref["y_exact"]).max() <= H.Y_TOL


@pytest.mark.parametrize("cfg", LS_CASES, ids=lambda c: c.name)
def test_least_squares_coefficients(cfg):
    H.note(f"case least squares {cfg.name}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    got = H.run_gpu(cfg, inp, coefficients="least_squares")
    ref = H.run_oracle(cfg, inp, want_ls=True)
    check_least_squares(cfg, got, ref)


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_least_squares_workload_sampled(name):
    """A workload at full size (C3: N=256, H=32, 128x128, W=8, r=8) with least-squares
    coefficients, as bench.py times it; 40 sampled units, every step and window."""
    cfg = workloads.get(name)
    H.note(f"case least squares {name} (sampled units)")
    inp = H.Inputs(cfg, workloads.sample_units(cfg, 40), cfg.steps)
    got = H.run_gpu(cfg, inp, coefficients="least_squares")
    ref = H.run_oracle(cfg, inp, want_ls=True)
    check_least_squares(cfg, got, ref)


@pytest.mark.parametrize("r", [8, 12])
def test_least_squares_low_rank_state(r):
    """A rank-2 window-start state: its sketch rows span two directions, so r - 2 rows are
    dropped by the factorisation (r = 8 in registers, r = 12 through LDS) and the first
    window's read, the projection of the exact read on that span, equals the exact read."""
    cfg = small("gdn", N=2, Hh=3, W=4, T=8, r=r)
    H.note(f"case least squares, rank-2 state, r={r}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    rng = np.random.default_rng([0x2A, r])
    U = rng.standard_normal((cfg.units, cfg.d_k, 2))
    V = rng.standard_normal((cfg.units, 2, cfg.d_v))
    S0 = (0.1 * U @ V).astype(np.float32)
    inp.S0.copy_(torch.from_numpy(S0.reshape(inp.S0.shape)))
    inp.host_S0 = S0.astype(np.float64)
    got = H.run_gpu(cfg, inp, coefficients="least_squares")
    ref = H.run_oracle(cfg, inp, want_ls=True)
    check_least_squares(cfg, got, ref)
    Q0 = got["Sk"][0]                                   # the first window's stored rows
    n_rows = (np.linalg.norm(Q0, axis=-1) > 0.5).sum(axis=-1)
    assert np.all(n_rows == 2), f"kept rows per unit: {n_rows}"
    e = H.rel_rows(got["y_sketch"][:cfg.window], got["y_full"][:cfg.window])
    assert e.max() <= H.Y_TOL, f"first window: least-squares read off the exact read by {e.max():.2e}"


def test_least_squares_ill_conditioned_sketch():
    """A window-start state that is rank one up to a 1e-4 perturbation: its eight sketch rows
    are dependent to about 1e-4, far from the drop threshold on most rows but near it. The
    stored rows must still be orthonormal to 1e-5 (a forward substitution through rows of Q
    rounded to fp32 loses about 5e-5 here)."""
    cfg = small("gdn", N=2, Hh=3, W=4, T=8, r=8)
    H.note("case least squares, ill-conditioned sketch")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    rng = np.random.default_rng(0x111)
    u = rng.standard_normal((cfg.units, cfg.d_k, 1))
    v = rng.standard_normal((cfg.units, 1, cfg.d_v))
    S0 = (0.1 * (u @ v + 1e-4 * rng.standard_normal((cfg.units, cfg.d_k, cfg.d_v)))).astype(np.float32)
    inp.S0.copy_(torch.from_numpy(S0.reshape(inp.S0.shape)))
    inp.host_S0 = S0.astype(np.float64)
    got = H.run_gpu(cfg, inp, coefficients="least_squares")
    ref = H.run_oracle(cfg, inp, want_ls=True)
    check_least_squares(cfg, got, ref)


def test_least_squares_zero_state():
    """A zero state has a zero sketch: every row is dropped and the read is the window
    term alone, equal to the exact read within the first window."""
    cfg = small("gdn", N=2, Hh=3, W=4, T=4)
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    inp.S0.zero_()
    inp.host_S0[:] = 0.0
    got = H.run_gpu(cfg, inp, coefficients="least_squares")
    assert np.all(got["Sk"][0] == 0.0)
    e = H.rel_rows(got["y_sketch"], got["y_full"])
    assert e.max() <= H.Y_TOL, f"{e.max():.2e}"


@pytest.mark.parametrize("rule", ["gdn", "kda"])
def test_graph_replay_matches_eager(rule):
    """One window of decode steps (fused appends, sketch reads, the update with the refresh)
    captured in a HIP graph gives, on every replay, exactly the eager outputs, state and
    sketch. Between replays the state is restored and the sketch refreshed eagerly."""
    cfg = small(rule, N=8, Hh=4, W=4, T=4)
    H.note(f"case graph replay {rule}")
    inp = H.Inputs(cfg, np.arange(cfg.units), cfg.steps)
    d = H.dims_of(cfg)
    W = cfg.window

    def fresh():
        state = inp.S0.clone()
        dec = WindowedDecoder(d, state, inp.basis, read="sketch")
        dec.refresh()
        return state, dec

    ys = [torch.empty((cfg.batch, cfg.heads, cfg.d_v), device="cuda") for _ in range(W)]
    state_e, dec_e = fresh()
    for t in range(W):
        dec_e.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t], y=ys[t])
    torch.cuda.synchronize()
    want_y = [y.clone() for y in ys]
    want_S, want_Sk = state_e.clone(), dec_e.sketch.clone()

    state_g, dec_g = fresh()
    gy = [torch.empty_like(y) for y in ys]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(W):
            dec_g.step(inp.q[t], inp.k[t], inp.v[t], inp.decay[t], inp.beta[t], y=gy[t])
    torch.cuda.synchronize()
    for rep in range(3):
        state_g.copy_(inp.S0)
        dec_g.tau = 0
        dec_g.refresh()
        torch.cuda.synchronize()
        for y in gy:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t in range(W):
            assert torch.equal(gy[t], want_y[t]), f"replay {rep}: step {t} output differs"
        assert torch.equal(state_g, want_S), f"replay {rep}: state differs"
        assert torch.equal(dec_g.sketch, want_Sk), f"replay {rep}: sketch differs"


@pytest.mark.parametrize("shape,n_tiles", [(0, 5), (0, 16), (1, 6)])
def test_stream_probe_in_place(shape, n_tiles):
    """The bandwidth probe reads and writes every value of its buffer in place (times 1.0):
    a guard band on both sides stays untouched."""
    H.note(f"stream_probe shape={shape} n_tiles={n_tiles}")
    g = torch.Generator(device="cuda").manual_seed(7)
    buf = torch.randn((n_tiles + 2) * 16384, device="cuda", generator=g)
    before = buf.clone()
    inner = buf[16384:(n_tiles + 1) * 16384]
    ssm.stream_probe(inner, n_tiles, shape)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def _staggered_run(cfg, T, units, single_launch: bool):
    """The staggered schedule at full size: sequence n joins at step n mod W; every step reads
    all rows at their own window positions (identity slots, padding rows at tau = 0 before
    they join) and updates the N/W rows whose window just filled. single_launch: one
    ssm_decode_step_varlen per step (double-buffered sketch, parity per row); else a varlen
    read and a varlen update per step. Returns the sampled units' outputs per local step and
    the final state and current sketch of those units."""
    N, Hh, dk, dv, W = cfg.batch, cfg.heads, cfg.d_k, cfg.d_v, cfg.window
    join = np.arange(N) % W
    S0 = workloads.initial_state(cfg)
    B = workloads.basis(cfg)
    with ThreadPoolExecutor(8) as ex:                            # local step j, row n
        local = list(ex.map(lambda j: workloads.step_inputs(cfg, j), range(T)))
    dev = "cuda"
    state = H._to_dev(S0, dev).view(N, Hh, dk, dv).clone()
    basis = H._to_dev(B, dev)
    d = H.dims_of(cfg)
    sketch = [torch.empty((N, Hh, cfg.rank, dv), device=dev) for _ in range(2)]
    tin = torch.bfloat16 if cfg.in_dtype == "bf16" else torch.float32
    kb = torch.zeros((N, Hh, W, dk), device=dev, dtype=tin)
    vb = torch.zeros((N, Hh, W, dv), device=dev, dtype=tin)
    db = torch.zeros(workloads.decay_shape(cfg, (N, Hh, W)), device=dev)
    bb = torch.zeros((N, Hh, W), device=dev) if cfg.has_beta else None
    ssm.window_update_refresh(d, state, sketch[0], basis, None, None, None, None, 0)
    idx = torch.as_tensor(units, device=dev)
    sentinel = 777.0
    y = torch.empty((N, Hh, dv), device=dev)
    got = {int(u): [] for u in units}
    rows = np.arange(N)

    def mix(field, t):
        """Global step t's input: row n from sequence n's local step t - join[n] (zeros
        before it joins); None for a field the rule does not have."""
        if getattr(local[0], field) is None:
            return None
        out = np.zeros_like(getattr(local[0], field))
        for s in range(W):
            live = (join == s) & (t >= s)
            if live.any():
                out[live] = getattr(local[t - s], field)[live]
        return out

    for t in range(T):
        tau = np.where(t >= join, (t - join) % W + 1, 0).astype(np.int32)
        parity = np.where(t >= join, ((t - join) // W) % 2, 0).astype(np.int32)
        y.fill_(sentinel)
        td = lambda f: None if mix(f, t) is None else H._to_dev(np.ascontiguousarray(mix(f, t)),
                                                               dev)
        ups = rows[tau == W].astype(np.int32)
        if single_launch:
            ssm.decode_step_varlen(d, N, None, H._to_dev(tau, dev), H._to_dev(parity, dev),
                                   len(ups), H._to_dev(ups, dev) if len(ups) else None, state,
                                   sketch[0], sketch[1], basis, td("q"), td("k"), td("v"),
                                   td("decay"), td("beta"), kb, vb, db, bb, y)
        else:
            ssm.sketch_decode_step_varlen(d, N, None, H._to_dev(tau, dev), sketch[0], basis,
                                          td("q"), kb, vb, db, bb, y, k_t=td("k"), v_t=td("v"),
                                          decay_t=td("decay"), beta_t=td("beta"))
            if len(ups):
                ssm.window_update_refresh_varlen(H.dims_of(cfg.with_(batch=len(ups))), N,
                                                 H._to_dev(ups, dev),
                                                 H._to_dev(np.full(len(ups), W, np.int32), dev),
                                                 state, sketch[0], basis, kb, vb, db, bb)
        yc = y.view(N * Hh, dv)[idx].cpu().double().numpy()
        for i, u in enumerate(units):
            n = u // Hh
            if t >= join[n]:
                got[int(u)].append(yc[i])
            else:
                assert (yc[i] == sentinel).all(), f"padding row {n} written at step {t}"
    torch.cuda.synchronize()
    S_end = state.view(N * Hh, dk, dv)[idx].cpu().double().numpy()
    # each sequence's current sketch: after its last full window (single launch: the buffer
    # its parity selects next)
    K = [sk.view(N * Hh, cfg.rank, dv)[idx].cpu().double().numpy() for sk in sketch]
    nwin = (T - join[units // Hh]) // W
    cur = nwin % 2 if single_launch else np.zeros_like(nwin)
    K_end = np.where(cur[:, None, None] == 1, K[1], K[0])
    return got, S_end, K_end, S0, B, local, join


def _staggered_check(cfg, T, units, got, S_end, K_end, S0, B, local, join):
    import oracle
    N, Hh, dk, dv, W = cfg.batch, cfg.heads, cfg.d_k, cfg.d_v, cfg.window
    worst = 0.0
    for s in range(W):
        sel = [i for i, u in enumerate(units) if join[u // Hh] == s]
        if not sel:
            continue
        us = units[sel]
        Tn = T - s
        flat = lambda x, e: x.reshape((N * Hh,) + ((e,) if e else ()))[us]
        pick = lambda f, e: np.stack([flat(getattr(local[j], f), e) for j in range(Tn)])
        ref = oracle.run(cfg.rule, S0.reshape(N * Hh, dk, dv)[us].astype(np.float64),
                         B[us % Hh].astype(np.float64), workloads.widen(pick("q", dk)),
                         workloads.widen(pick("k", dk)), workloads.widen(pick("v", dv)),
                         pick("decay", dk if cfg.per_channel_decay else 0).astype(np.float64),
                         pick("beta", 0).astype(np.float64) if cfg.has_beta else None, W)
        g = np.stack([np.stack(got[int(u)]) for u in us], axis=1)    # [Tn][U][dv]
        e = H.rel_rows(g, ref["y_sketch"])
        worst = max(worst, float(e.max()))
        assert e.max() <= H.Y_TOL, f"phase {s}: sketch read {e.max():.3e}"
        nw = Tn // W
        H.assert_mats(S_end[sel][None], ref["S_win"][nw][None], H.S_TOL, f"phase {s}: state")
        H.assert_mats(K_end[sel][None], ref["Sk"][nw][None], H.S_TOL, f"phase {s}: sketch")
    return worst


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_staggered_windows_workload_sampled(name):
    """A workload at full size (C3: N=256, H=32, 128x128, W=8, r=8) on the staggered schedule
    bench.py times: sequence n joins at step n mod W, so from step W - 1 on every step reads
    all rows at their own window positions (one varlen read, identity slots) and updates the
    N/W rows whose window just filled (one varlen update). Rows that have not joined are
    padding (tau = 0) and keep their output. 40 sampled units are checked against the oracle
    over their local steps: every output, and the final state and sketch."""
    cfg = workloads.get(name)
    T = 64 + cfg.window - 1                      # the last joiner still runs 64 local steps
    H.note(f"case staggered windows {name} (sampled units)")
    units = workloads.sample_units(cfg, 40)
    res = _staggered_run(cfg, T, units, single_launch=False)
    worst = _staggered_check(cfg, T, units, *res)
    H.note(f"staggered {name}: worst sketch-read error {worst:.2e}")


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_single_launch_step_staggered_workload_sampled(name):
    """The same staggered schedule through ssm_decode_step_varlen, one launch per step (the
    read of every row, the update of the rows whose window fills, a double-buffered sketch
    chosen per row by parity), as bench.py times it: against the oracle, and bit for bit
    equal to the two-launch schedule (same arithmetic; the update takes the window's newest
    token from the step's inputs instead of the buffer, the same bits)."""
    cfg = workloads.get(name)
    T = 64 + cfg.window - 1
    H.note(f"case single-launch staggered step {name} (sampled units)")
    units = workloads.sample_units(cfg, 40)
    one = _staggered_run(cfg, T, units, single_launch=True)
    worst = _staggered_check(cfg, T, units, *one)
    two = _staggered_run(cfg, T, units, single_launch=False)
    for u in units:
        assert np.array_equal(np.stack(one[0][int(u)]), np.stack(two[0][int(u)])), f"unit {u}"
    assert np.array_equal(one[1], two[1]) and np.array_equal(one[2], two[2])
    H.note(f"single-launch staggered {name}: worst sketch-read error {worst:.2e}")


@pytest.mark.parametrize("rule,sketch_dtype,d_v,in_dtype", [
    ("mamba2", "f32", 64, "bf16"), ("gdn", "f32", 64, "bf16"), ("kda", "f32", 64, "bf16"),
    ("mamba2", "bf16", 64, "bf16"), ("gdn", "bf16", 64, "bf16"), ("kda", "bf16", 64, "bf16"),
    ("gdn", "f32", 16, "bf16"), ("kda", "bf16", 16, "bf16"),
    ("mamba2", "f32", 16, "f32"), ("gdn", "bf16", 64, "f32"), ("kda", "f32", 64, "f32")])
def test_single_launch_step_continuous_batching(rule, sketch_dtype, d_v, in_dtype):
    """ssm_decode_step_varlen with sequences joining at different steps into permuted pool
    slots, reversed row order and a padding row (tau = 0, its output left untouched): every
    sequence against its own oracle run (outputs every step, state and current sketch at the
    end). A bf16 sketch is compared with the oracle's rounding through oracle values only,
    as in the harness (the stored element within its rounding window; the read beyond what
    those windows allow within the fp32 tolerance)."""
    import oracle
    W, T = 4, 14
    joins = [0, 1, 2, 3, 5, 6]
    slots = [5, 0, 7, 2, 3, 6]
    P = 8                                      # pool size
    cfg = small(rule, in_dtype, d_k=64, d_v=d_v, W=W, r=8, N=len(joins), Hh=3, T=T)
    H.note(f"case single-launch step, continuous batching {rule} {sketch_dtype} d_v={d_v} "
           f"{in_dtype} inputs")
    Hh, dk, dv = cfg.heads, cfg.d_k, cfg.d_v
    S0 = np.concatenate([workloads.initial_state(cfg, [n]) for n in range(len(joins))])
    B = workloads.basis(cfg)
    steps = [workloads.step_inputs(cfg, j) for j in range(T)]   # local step j, row n = sequence n
    d_pool = H.dims_of(cfg.with_(batch=P), sketch_dtype)
    dev = "cuda"
    tin = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    skt = torch.bfloat16 if sketch_dtype == "bf16" else torch.float32

    def td(x):
        return None if x is None else H._to_dev(np.ascontiguousarray(x), dev)

    state = torch.zeros((P, Hh, dk, dv), device=dev)
    sketch = [torch.zeros((P, Hh, cfg.rank, dv), device=dev, dtype=skt) for _ in range(2)]
    kb = torch.zeros((P, Hh, W, dk), device=dev, dtype=tin)
    vb = torch.zeros((P, Hh, W, dv), device=dev, dtype=tin)
    dshape = (P, Hh, W, dk) if rule == "kda" else (P, Hh, W)
    db = torch.zeros(dshape, device=dev)
    bb = torch.zeros((P, Hh, W), device=dev) if rule != "mamba2" else None
    basis = td(B)
    got_y = {n: [] for n in range(len(joins))}
    sentinel = 777.0
    for t in range(T):
        joining = [n for n in range(len(joins)) if joins[n] == t]
        for n in joining:
            state[slots[n]] = torch.from_numpy(S0[n]).to(dev)
        if joining:   # refresh-only pass into buffer 0 for the sequences that just joined
            dj = H.dims_of(cfg.with_(batch=len(joining)), sketch_dtype)
            ssm.window_update_refresh_varlen(
                dj, P, td(np.array([slots[n] for n in joining], np.int32)),
                td(np.zeros(len(joining), np.int32)), state, sketch[0], basis, kb, vb, db, bb)
        active = [n for n in range(len(joins)) if joins[n] <= t][::-1]   # reversed row order
        rows = active + [None]                                          # + one padding row
        tau = [((t - joins[n]) % W) + 1 if n is not None else 0 for n in rows]
        par = [((t - joins[n]) // W) % 2 if n is not None else 0 for n in rows]
        slot_rows = [slots[n] if n is not None else 1 for n in rows]
        pick = lambda x, n: x[n] if n is not None else np.zeros_like(x[0])
        loc = lambda n: t - joins[n] if n is not None else 0
        q = np.stack([pick(steps[loc(n)].q, n) for n in rows])
        k = np.stack([pick(steps[loc(n)].k, n) for n in rows])
        v = np.stack([pick(steps[loc(n)].v, n) for n in rows])
        dc = np.stack([pick(steps[loc(n)].decay, n) for n in rows])
        bt = (np.stack([pick(steps[loc(n)].beta, n) for n in rows]) if rule != "mamba2" else None)
        ups = np.array([i for i in range(len(active)) if tau[i] == W], np.int32)
        dr = H.dims_of(cfg.with_(batch=len(rows)), sketch_dtype)
        y = torch.full((len(rows), Hh, dv), sentinel, device=dev)
        ssm.decode_step_varlen(dr, P, td(np.array(slot_rows, np.int32)),
                               td(np.array(tau, np.int32)), td(np.array(par, np.int32)),
                               len(ups), td(ups) if len(ups) else None, state, sketch[0],
                               sketch[1], basis, td(q), td(k), td(v), td(dc), td(bt), kb, vb, db,
                               bb, y)
        yc = y.cpu().double().numpy()
        assert (yc[-1] == sentinel).all(), "padding row was written"
        for i, n in enumerate(active):
            got_y[n].append(yc[i])
    torch.cuda.synchronize()
    for n in range(len(joins)):
        Tn = T - joins[n]
        wid = lambda x, e: x.reshape((cfg.batch, Hh) + ((e,) if e else ()))[n]
        hq = np.stack([workloads.widen(wid(steps[j].q, dk)) for j in range(Tn)])
        hk = np.stack([workloads.widen(wid(steps[j].k, dk)) for j in range(Tn)])
        hv = np.stack([workloads.widen(wid(steps[j].v, dv)) for j in range(Tn)])
        hd = np.stack([wid(steps[j].decay, dk if rule == "kda" else 0) for j in range(Tn)]).astype(np.float64)
        hb = (np.stack([wid(steps[j].beta, 0) for j in range(Tn)]).astype(np.float64)
              if rule != "mamba2" else None)
        bf = sketch_dtype == "bf16"
        Bf = B.astype(np.float64)
        ref = oracle.run(rule, S0[n].astype(np.float64), Bf, hq, hk, hv, hd, hb, W,
                         sketch_bf16=bf, want_ls=bf)
        nw = Tn // W
        gy = np.stack(got_y[n])
        gK = sketch[nw % 2][slots[n]].float().cpu().double().numpy()
        if bf:
            # oracle values only: the stored element lies in its rounding window around the
            # unrounded sketch, and the read may move by what those windows allow
            ref_exact = oracle.run(rule, S0[n].astype(np.float64), Bf, hq, hk, hv, hd, hb, W)
            c_sub = cfg.with_(batch=1)
            slack = H.bf16_read_slack(c_sub, ref, ref_exact, Bf)
            e = H.rel_diff_rows(np.maximum(np.abs(gy - ref["y_sketch"]) - slack, 0.0),
                                ref["y_sketch"])
            lo, hi = H.bf16_window(ref_exact["Sk"][nw][None], H.S_TOL)
            assert np.all((gK[None] >= lo) & (gK[None] <= hi)), f"sequence {n}: bf16 sketch"
        else:
            e = H.rel_rows(gy, ref["y_sketch"])
            H.assert_mats(gK[None, None], ref["Sk"][nw][None, None], H.S_TOL, f"sequence {n}: sketch")
        assert e.max() <= H.Y_TOL, f"sequence {n}: sketch read {e.max():.3e}"
        gS = state[slots[n]].cpu().double().numpy()
        H.assert_mats(gS[None, None], ref["S_win"][nw][None, None], H.S_TOL, f"sequence {n}: state")
    # slots 4 and 1 were never assigned to a sequence: untouched
    assert torch.count_nonzero(state[4]) == 0 and torch.count_nonzero(state[1]) == 0
