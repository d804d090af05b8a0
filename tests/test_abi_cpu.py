"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects bad arguments on the host before anything is enqueued.

Every call below is built to fail validation (or to be a declared no-op), so
no kernel is ever launched; the fake device addresses are never dereferenced.
"""
import ctypes
import shutil
import subprocess

import pytest

import sketched_recurrent_state_amd as ssm

A = 1 << 32  # a 16-byte aligned fake device address (never dereferenced)


def dims(rule="gdn", in_dtype="bf16", batch=2, heads=3, d_k=32, d_v=64, window=4, rank=4):
    return ssm.Dims.make(rule, in_dtype, batch, heads, d_k, d_v, window, rank)


def addrs(n, gap=1 << 28):
    """n disjoint, aligned fake addresses."""
    return [A + i * gap for i in range(n)]


def status_of(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except ssm.SSMError as e:
        return e.status, e.detail
    return 0, ""


def test_every_declared_symbol_is_exported():
    names = ssm.declared_symbols()
    assert set(names) >= {"ssm_abi_version", "ssm_status_string", "ssm_last_error",
                          "ssm_buffer_append", "ssm_window_update_refresh",
                          "ssm_sketch_decode_step", "ssm_full_read_decode_step"}
    lib = ssm.library()
    for n in names:
        assert hasattr(lib, n), n
    if shutil.which("nm"):
        out = subprocess.run(["nm", "-D", "--defined-only", ssm.LIB_PATH], capture_output=True,
                             text=True, check=True).stdout
        exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
        assert set(names) <= exported


def test_version_and_status_strings():
    assert ssm.abi_version() == 5
    lib = ssm.library()
    for code in range(7):
        assert lib.ssm_status_string(code).decode()
    assert lib.ssm_status_string(99).decode() == "unknown status"


def test_null_dims():
    lib = ssm.library()
    st = lib.ssm_window_update_refresh(None, A, A, A, A, A, A, A, 1, None)
    assert st == 1 and "dims is NULL" in lib.ssm_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("rule", 3, 4), ("rule", -1, 4), ("in_dtype", 2, 4),
    ("batch", -1, 2), ("heads", 0, 2), ("d_k", 48, 2), ("d_k", 256, 2), ("d_v", 8, 2),
    ("d_v", 256, 2), ("window", 0, 2), ("window", 17, 2), ("rank", 0, 2), ("rank", 33, 2),
    ("sketch_dtype", 2, 4), ("sketch_dtype", -1, 4),
])
def test_bad_dims(field, value, code):
    d = dims()
    setattr(d, field, value)
    p = addrs(8)
    st, msg = status_of(ssm.window_update_refresh, d, *p[:7], 1)
    assert st == code, msg
    assert field.replace("_", "") in msg.replace("_", "").lower() or field in msg


def test_rank_above_d_k():
    d = dims(d_k=16, rank=17)
    st, msg = status_of(ssm.window_update_refresh, d, *addrs(7), 1)
    assert st == 2 and "rank" in msg


def test_too_many_units():
    d = dims(batch=1 << 20, heads=16)
    st, msg = status_of(ssm.window_update_refresh, d, *addrs(7), 1)
    assert st == 2 and "batch*heads" in msg


@pytest.mark.parametrize("n_tokens", [-1, 5])
def test_n_tokens_range(n_tokens):
    st, msg = status_of(ssm.window_update_refresh, dims(window=4), *addrs(7), n_tokens)
    assert st == 4 and "n_tokens" in msg


@pytest.mark.parametrize("tau", [0, 5])
def test_tau_range(tau):
    p = addrs(8)
    st, _ = status_of(ssm.sketch_decode_step, dims(window=4), p[0], p[1], p[2], p[3], p[4], p[5],
                      p[6], tau, p[7])
    assert st == 4
    st, _ = status_of(ssm.full_read_decode_step, dims(window=4), p[0], p[2], p[3], p[4], p[5], p[6],
                      tau, p[7])
    assert st == 4


@pytest.mark.parametrize("slot", [-1, 4])
def test_slot_range(slot):
    st, msg = status_of(ssm.buffer_append, dims(window=4), *addrs(8), slot)
    assert st == 4 and "slot" in msg


def test_empty_batch_is_a_noop():
    # batch = 0: nothing to do, no pointer is looked at, nothing is launched
    d = dims(batch=0)
    assert status_of(ssm.window_update_refresh, d, None, None, None, None, None, None, None, 2)[0] == 0
    assert status_of(ssm.sketch_decode_step, d, None, None, None, None, None, None, None, 1, None)[0] == 0
    assert status_of(ssm.full_read_decode_step, d, None, None, None, None, None, None, 1, None)[0] == 0
    assert status_of(ssm.buffer_append, d, None, None, None, None, None, None, None, None, 0)[0] == 0


def test_nothing_to_do_is_a_noop():
    # no tokens and no sketch requested: no launch
    p = addrs(7)
    assert status_of(ssm.window_update_refresh, dims(), p[0], None, None, None, None, None, None, 0)[0] == 0


def test_null_pointers():
    p = addrs(12)
    d = dims()
    st, msg = status_of(ssm.window_update_refresh, d, None, p[1], p[2], p[3], p[4], p[5], p[6], 1)
    assert st == 1 and "state" in msg
    st, msg = status_of(ssm.window_update_refresh, d, p[0], p[1], None, p[3], p[4], p[5], p[6], 1)
    assert st == 1 and "basis" in msg
    st, msg = status_of(ssm.window_update_refresh, d, p[0], p[1], p[2], None, p[4], p[5], p[6], 1)
    assert st == 1 and "k_buf" in msg
    st, msg = status_of(ssm.window_update_refresh, d, p[0], p[1], p[2], p[3], p[4], p[5], None, 1)
    assert st == 1 and "beta_buf" in msg
    st, msg = status_of(ssm.sketch_decode_step, d, p[0], p[1], None, p[3], p[4], p[5], p[6], 1, p[7])
    assert st == 1 and "q" in msg
    st, msg = status_of(ssm.sketch_decode_step, d, p[0], p[1], p[2], p[3], p[4], p[5], p[6], 1, None)
    assert st == 1 and "y" in msg
    st, msg = status_of(ssm.full_read_decode_step, d, None, p[2], p[3], p[4], p[5], p[6], 1, p[7])
    assert st == 1 and "state" in msg


def test_beta_rules():
    p = addrs(8)
    # Mamba-2 takes no beta
    st, msg = status_of(ssm.window_update_refresh, dims(rule="mamba2"), *p[:7], 1)
    assert st == 4 and "Mamba-2" in msg
    # the delta rules need it
    st, msg = status_of(ssm.buffer_append, dims(rule="kda"), p[0], p[1], p[2], None, *p[4:8], 0)
    assert st == 1 and "beta_t" in msg


def test_fused_token_all_or_nothing():
    p = addrs(12)
    d = dims()
    st, msg = status_of(ssm.sketch_decode_step, d, *p[:7], 1, p[7], v_t=p[8])
    assert st == 4 and "k_t is NULL" in msg
    st, msg = status_of(ssm.sketch_decode_step, d, *p[:7], 1, p[7], k_t=p[8], v_t=p[9])
    assert st == 1 and "decay_t" in msg


def test_alignment():
    p = addrs(8)
    st, msg = status_of(ssm.window_update_refresh, dims(), p[0] + 8, *p[1:7], 1)
    assert st == 3 and "state" in msg
    st, msg = status_of(ssm.sketch_decode_step, dims(), *p[:6], p[6] + 4, 1, p[7])
    assert st == 3 and "beta_buf" in msg


def test_aliasing():
    p = addrs(8)
    # sketch placed inside the state
    st, msg = status_of(ssm.window_update_refresh, dims(), p[0], p[0] + 256, *p[2:7], 1)
    assert st == 5 and "overlaps" in msg
    # y on top of q
    st, msg = status_of(ssm.sketch_decode_step, dims(), p[0], p[1], p[2], *p[3:7], 1, p[2])
    assert st == 5 and "overlaps" in msg
    # fused append writes the buffers: they must not overlap the token inputs
    st, msg = status_of(ssm.sketch_decode_step, dims(), *p[:7], 1, p[7], k_t=p[3], v_t=A + (40 << 28),
                        decay_t=A + (41 << 28), beta_t=A + (42 << 28))
    assert st == 5 and "overlaps" in msg
    # unfused reads of the same buffer from two arguments are fine to check: inputs may overlap
    d = dims(rule="mamba2")
    st, msg = status_of(ssm.full_read_decode_step, d, p[0], p[1], p[1], p[1], p[1], None, 1, p[1])
    assert st == 5  # but y may not overlap them


def test_bf16_sketch_is_sized_in_bf16():
    # dims(): 6 units x rank 4 x d_v 64 -> the sketch is 6144 bytes in fp32, 3072 in bf16.
    # The basis sits 3072 bytes after the sketch and k_buf overlaps the sketch's first half,
    # so the first overlap found names the basis for an fp32 sketch and k_buf for a bf16 one.
    # Either way validation fails before anything is launched.
    s = A + (8 << 28)
    state, basis, kbuf = A, s + 3072, s + 3056
    vbuf, dbuf, bbuf = A + (9 << 28), A + (10 << 28), A + (11 << 28)
    st, msg = status_of(ssm.window_update_refresh, dims(), state, s, basis, kbuf, vbuf, dbuf,
                        bbuf, 2)
    assert st == 5 and "sketch overlaps basis" in msg, msg
    d = ssm.Dims.make("gdn", "bf16", 2, 3, 32, 64, 4, 4, sketch_dtype="bf16")
    assert d.sketch_dtype == ssm.SKETCH_BF16
    st, msg = status_of(ssm.window_update_refresh, d, state, s, basis, kbuf, vbuf, dbuf, bbuf, 2)
    assert st == 5 and "sketch overlaps k_buf" in msg, msg


def test_last_error_is_thread_local_and_cleared():
    import threading
    lib = ssm.library()
    status_of(ssm.window_update_refresh, dims(window=4), *addrs(7), 9)
    assert "n_tokens" in lib.ssm_last_error().decode()
    seen = {}

    def other():
        seen["msg"] = lib.ssm_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    # a successful (no-op) call clears it
    assert status_of(ssm.window_update_refresh, dims(batch=0), *addrs(7), 0)[0] == 0
    assert lib.ssm_last_error().decode() == ""


def test_binding_checks_tensor_sizes_on_host():
    torch = pytest.importorskip("torch")
    # CPU tensors are rejected before anything reaches the library
    d = dims()
    with pytest.raises(ValueError, match="device tensor"):
        ssm.window_update_refresh(d, torch.zeros(4), None, None, None, None, None, None, 0)


def test_one_hip_runtime_in_the_process():
    """The library shares PyTorch's HIP runtime: two runtimes in one process
    leave the second one without a device."""
    import os
    maps = open("/proc/self/maps").read().splitlines()
    hip = {os.path.realpath(l.split()[-1]) for l in maps if "libamdhip64" in l}
    hsa = {os.path.realpath(l.split()[-1]) for l in maps if "libhsa-runtime64" in l}
    assert len(hip) == 1, hip
    assert len(hsa) <= 1, hsa


def test_recurrent_step_validation():
    p = addrs(8)
    d = dims()
    st, msg = status_of(ssm.recurrent_decode_step, d, None, *p[1:7])
    assert st == 1 and "state" in msg
    st, msg = status_of(ssm.recurrent_decode_step, d, p[0], p[1], None, p[3], p[4], p[5], p[6])
    assert st == 1 and "k_t" in msg
    st, msg = status_of(ssm.recurrent_decode_step, dims(rule="mamba2"), *p[:7])
    assert st == 4 and "Mamba-2" in msg
    st, msg = status_of(ssm.recurrent_decode_step, d, p[0], p[1], p[2], p[3], p[4], p[5], p[0] + 64)
    assert st == 5 and "overlaps" in msg
    assert status_of(ssm.recurrent_decode_step, dims(batch=0), *([None] * 7))[0] == 0


def test_rank_table_validation():
    p = addrs(8)
    d = dims(heads=3, d_k=32)
    # a valid table passes the table checks and stops at the NULL state
    st, msg = status_of(ssm.window_update_refresh_ranked, d, [0, 2, 5, 9], None, *p[1:7], 1)
    assert st == 1 and "state" in msg
    st, msg = status_of(ssm.window_update_refresh_ranked, d, [1, 2, 5, 9], *p[:7], 1)
    assert st == 4 and "rank_offsets[0]" in msg
    st, msg = status_of(ssm.window_update_refresh_ranked, d, [0, 2, 2, 9], *p[:7], 1)
    assert st == 4 and "head 1 has rank 0" in msg
    st, msg = status_of(ssm.sketch_decode_step_ranked, d, [0, 2, 40, 41], *p[:7], 1, p[7])
    assert st == 4 and "head 1 has rank 38" in msg
    with pytest.raises(ValueError, match="heads \\+ 1"):
        ssm.window_update_refresh_ranked(d, [0, 1, 2, 3, 4], *p[:7], 1)
    big = dims(heads=300, d_k=32)
    st, msg = status_of(ssm.window_update_refresh_ranked, big, [1] * 300, *p[:7], 1)
    assert st == 2 and "heads" in msg
    # sizes follow the table: a sketch that overlaps the state under the table's size is caught
    st, msg = status_of(ssm.window_update_refresh_ranked, d, [0, 2, 5, 9], p[0], p[0] + 2 * 3 * 32 * 64 * 4 - 16,
                        *p[2:7], 1)
    assert st == 5 and "overlaps" in msg


def test_varlen_validation():
    p = addrs(16)
    d = dims(batch=4)
    # 4 rows, 2 slots, no slot map: rejected
    st, msg = status_of(ssm.window_update_refresh_varlen, d, 2, None, p[0], *p[1:9])
    assert st == 2 and "slot map" in msg
    st, msg = status_of(ssm.window_update_refresh_varlen, d, 0, p[9], p[0], *p[1:9])
    assert st == 2 and "num_slots" in msg
    st, msg = status_of(ssm.sketch_decode_step_varlen, d, 8, None, None, *p[1:9])
    assert st == 1 and "tau" in msg
    # count arrays need 4-byte alignment only; state needs 16
    st, msg = status_of(ssm.window_update_refresh_varlen, d, 8, p[9] + 4, p[10] + 8, p[1] + 4, *p[2:9])
    assert st == 3 and "state" in msg
    # persistent arrays are sized by the pool: a sketch inside an 8-slot state overlaps it
    st, msg = status_of(ssm.window_update_refresh_varlen, d, 8, p[9], p[10], p[1],
                        p[1] + 8 * 3 * 32 * 64 * 4 - 64, *p[3:9])
    assert st == 5 and "state overlaps sketch" in msg
    # y may not overlap the tau array
    st, msg = status_of(ssm.sketch_decode_step_varlen, d, 8, p[9], p[10], p[1], p[2], p[3],
                        p[4], p[5], p[6], p[7], p[10])
    assert st == 5


def test_fit_basis_validation():
    p = addrs(4)
    d = dims()
    st, msg = status_of(ssm.fit_basis, d, None, 64, p[1])
    assert st == 1 and "samples" in msg
    st, msg = status_of(ssm.fit_basis, d, p[0], 64, None)
    assert st == 1 and "basis" in msg
    for n in (0, -3, (1 << 24) + 1):
        st, msg = status_of(ssm.fit_basis, d, p[0], n, p[1])
        assert st == 2 and "n_samples" in msg
    st, msg = status_of(ssm.fit_basis, d, p[0] + 8, 64, p[1])
    assert st == 3 and "samples" in msg
    # basis written inside the samples
    st, msg = status_of(ssm.fit_basis, d, p[0], 64, p[0] + 1024)
    assert st == 5 and "overlaps" in msg
    st, msg = status_of(ssm.fit_basis, dims(d_k=16, rank=17), p[0], 64, p[1])
    assert st == 2 and "rank" in msg


def test_stream_probe_validation():
    p = addrs(1)
    st, msg = status_of(ssm.stream_probe, None, 8, 0)
    assert st == 1 and "buf" in msg
    for shape in (-1, 2):
        st, msg = status_of(ssm.stream_probe, p[0], 8, shape)
        assert st == 4 and "shape" in msg
    for n in (0, -1, 1 << 24):
        st, msg = status_of(ssm.stream_probe, p[0], n, 0)
        assert st == 2 and "n_tiles" in msg
    st, msg = status_of(ssm.stream_probe, p[0], 7, 1)
    assert st == 2 and "even" in msg
    st, msg = status_of(ssm.stream_probe, p[0] + 4, 8, 0)
    assert st == 3 and "buf" in msg


def test_decode_step_varlen_validation():
    """The single-launch serving step: argument checks before anything is launched."""
    p = addrs(24)
    d = dims(batch=4)
    P = 8  # pool slots

    def call(**kw):
        a = dict(num_slots=P, slot=p[0], tau=p[1], parity=p[2], n_update=1, update_rows=p[3],
                 state=p[4], sketch0=p[5], sketch1=p[6], basis=p[7], q=p[8], k_t=p[9], v_t=p[10],
                 decay_t=p[11], beta_t=p[12], k_buf=p[13], v_buf=p[14], decay_buf=p[15],
                 beta_buf=p[16], y=p[17])
        a.update(kw)
        return status_of(ssm.decode_step_varlen, d, a.pop("num_slots"), a.pop("slot"),
                         a.pop("tau"), a.pop("parity"), a.pop("n_update"), a.pop("update_rows"),
                         **a)

    st, msg = call(parity=None)
    assert st == 1 and "parity" in msg
    st, msg = call(update_rows=None)
    assert st == 1 and "update_rows" in msg
    for n in (-1, 5):
        st, msg = call(n_update=n)
        assert st == 4 and "n_update" in msg
    st, msg = call(k_t=None, v_t=None, decay_t=None, beta_t=None)
    assert st == 1 and "k_t" in msg
    st, msg = call(sketch1=None)
    assert st == 1 and "sketch1" in msg
    # the two sketch buffers may not overlap each other (pool-sized: 8 slots x 3 heads x 4 x 64)
    st, msg = call(sketch1=p[5] + 8 * 3 * 4 * 64 * 4 - 16)
    assert st == 5 and "sketch0 overlaps sketch1" in msg
    # nor may y overlap the parity array
    st, msg = call(y=p[2])
    assert st == 5 and "overlaps" in msg
    st, msg = call(num_slots=2, slot=None)
    assert st == 2 and "slot map" in msg
    # no update rows: the list may be NULL; the call then stops at the NULL state
    st, msg = call(n_update=0, update_rows=None, state=None)
    assert st == 1 and "state" in msg
    # an empty batch is a no-op
    d0 = dims(batch=0)
    assert status_of(ssm.decode_step_varlen, d0, P, *([None] * 3), 0, *([None] * 16))[0] == 0


def test_least_squares_takes_d_v_16():
    """d_v = 16 is a supported shape for every entry point, the least-squares ones included:
    calls that are valid but for one NULL pointer stop at that pointer, not at the shape."""
    p = addrs(10)
    d = dims(d_v=16)
    st, msg = status_of(ssm.window_update_refresh_ls, d, None, *p[1:8], 1)
    assert st == 1 and "state" in msg
    st, msg = status_of(ssm.sketch_decode_step_ls, d, None, *p[1:7], 1, p[7])
    assert st == 1 and "sketch_q" in msg
    st, msg = status_of(ssm.window_update_refresh, d, None, *p[1:7], 1)
    assert st == 1 and "state" in msg
