"""SketchSSM windowed linear-attention decode for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libsketchssm.so`` (C ABI in
``include/sketchssm.h``). Each function here marshals its arguments and calls
the library entry point of the same name; every step of the decode path runs
in the library's HIP kernels. Tensors are PyTorch device tensors (PyTorch
provides memory and streams only) or raw device addresses as ``int``; a call
whose pointers and stream are all ``int`` goes straight to the library (the
library still checks the arguments, but not their sizes).

If the library has not been built this module raises on import: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

__all__ = [
    "Dims", "SSMError", "MAMBA2", "GDN", "KDA", "IN_BF16", "IN_F32", "RULES",
    "abi_version", "buffer_append", "window_update_refresh", "sketch_decode_step",
    "full_read_decode_step", "recurrent_decode_step", "window_update_refresh_ranked",
    "sketch_decode_step_ranked", "rank_offsets", "window_update_refresh_varlen",
    "sketch_decode_step_varlen", "decode_step_varlen", "window_update_refresh_ls",
    "sketch_decode_step_ls",
    "fit_basis", "stream_probe", "SKETCH_F32", "SKETCH_BF16", "LIB_PATH", "HEADER",
    "declared_symbols", "numel", "library",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsketchssm.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "sketchssm.h")

MAMBA2, GDN, KDA = 0, 1, 2
RULES = {"mamba2": MAMBA2, "gdn": GDN, "kda": KDA}
IN_BF16, IN_F32 = 0, 1
SKETCH_F32, SKETCH_BF16 = 0, 1

STATUS = {0: "SSM_OK", 1: "SSM_E_NULL", 2: "SSM_E_SHAPE", 3: "SSM_E_ALIGN", 4: "SSM_E_RANGE",
          5: "SSM_E_ALIAS", 6: "SSM_E_LAUNCH"}


class SSMError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class Dims(ctypes.Structure):
    """ssm_dims: rule, in_dtype, batch, heads, d_k, d_v, window, rank, sketch_dtype."""

    _fields_ = [(n, ctypes.c_int32) for n in
                ("rule", "in_dtype", "batch", "heads", "d_k", "d_v", "window", "rank",
                 "sketch_dtype")]

    @classmethod
    def make(cls, rule, in_dtype, batch, heads, d_k, d_v, window, rank,
             sketch_dtype="f32") -> "Dims":
        if isinstance(rule, str):
            rule = RULES[rule]
        if isinstance(in_dtype, str):
            in_dtype = {"bf16": IN_BF16, "f32": IN_F32}[in_dtype]
        if isinstance(sketch_dtype, str):
            sketch_dtype = {"f32": SKETCH_F32, "bf16": SKETCH_BF16}[sketch_dtype]
        return cls(rule, in_dtype, batch, heads, d_k, d_v, window, rank, sketch_dtype)

    def __repr__(self):
        return "Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


def _load():
    # The tensors handed to the library come from PyTorch's HIP runtime, and the
    # process must hold exactly one HIP runtime: load torch first so that the
    # library's libamdhip64.so.7 dependency resolves to the copy torch loaded.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python sketched_recurrent_state_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, dp = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(Dims)
    lib.ssm_abi_version.restype = i32
    lib.ssm_abi_version.argtypes = []
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_status_string.argtypes = [i32]
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_last_error.argtypes = []
    lib.ssm_buffer_append.restype = i32
    lib.ssm_buffer_append.argtypes = [dp] + [vp] * 8 + [i32, vp]
    lib.ssm_window_update_refresh.restype = i32
    lib.ssm_window_update_refresh.argtypes = [dp] + [vp] * 7 + [i32, vp]
    lib.ssm_sketch_decode_step.restype = i32
    lib.ssm_sketch_decode_step.argtypes = [dp] + [vp] * 11 + [i32, vp, vp]
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.ssm_window_update_refresh_ranked.restype = i32
    lib.ssm_window_update_refresh_ranked.argtypes = [dp, ip] + [vp] * 7 + [i32, vp]
    lib.ssm_sketch_decode_step_ranked.restype = i32
    lib.ssm_sketch_decode_step_ranked.argtypes = [dp, ip] + [vp] * 11 + [i32, vp, vp]
    lib.ssm_window_update_refresh_varlen.restype = i32
    lib.ssm_window_update_refresh_varlen.argtypes = [dp, i32] + [vp] * 9 + [vp]
    lib.ssm_sketch_decode_step_varlen.restype = i32
    lib.ssm_sketch_decode_step_varlen.argtypes = [dp, i32] + [vp] * 15
    lib.ssm_decode_step_varlen.restype = i32
    lib.ssm_decode_step_varlen.argtypes = [dp, i32, vp, vp, vp, i32] + [vp] * 15 + [vp]
    lib.ssm_recurrent_decode_step.restype = i32
    lib.ssm_recurrent_decode_step.argtypes = [dp] + [vp] * 7 + [vp]
    lib.ssm_full_read_decode_step.restype = i32
    lib.ssm_full_read_decode_step.argtypes = [dp] + [vp] * 10 + [i32, vp, vp]
    lib.ssm_window_update_refresh_ls.restype = i32
    lib.ssm_window_update_refresh_ls.argtypes = [dp] + [vp] * 8 + [i32, vp]
    lib.ssm_sketch_decode_step_ls.restype = i32
    lib.ssm_sketch_decode_step_ls.argtypes = [dp] + [vp] * 11 + [i32, vp, vp]
    lib.ssm_fit_basis.restype = i32
    lib.ssm_fit_basis.argtypes = [dp, vp, i32, vp, vp]
    lib.ssm_stream_probe.restype = i32
    lib.ssm_stream_probe.argtypes = [vp, ctypes.c_int64, i32, vp]
    return lib


_lib = _load()


def declared_symbols(header: str = HEADER):
    """Function names declared in the C header."""
    import re
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:ssm_status|int32_t|const char\*)\s+(ssm_\w+)\s*\(",
                                 text, re.M)))


def library():
    return _lib


def abi_version() -> int:
    return int(_lib.ssm_abi_version())


# ----------------------------------------------------------------------------
# marshalling
# ----------------------------------------------------------------------------
Ptr = Union["torch.Tensor", int, None]  # noqa: F821


def numel(d: Dims) -> dict:
    """Element count of every array argument for these dimensions."""
    U = d.batch * d.heads
    dstr = d.d_k if d.rule == KDA else 1
    return {
        "state": U * d.d_k * d.d_v, "sketch": U * d.rank * d.d_v, "basis": d.heads * d.rank * d.d_k,
        "read_map": U * d.rank * d.d_k,
        "k_buf": U * d.window * d.d_k, "v_buf": U * d.window * d.d_v,
        "decay_buf": U * d.window * dstr, "beta_buf": U * d.window,
        "q": U * d.d_k, "k_t": U * d.d_k, "v_t": U * d.d_v, "decay_t": U * dstr, "beta_t": U,
        "y": U * d.d_v,
    }


def _addr(x: Ptr, name: str, dtype=None, count: Optional[int] = None) -> Optional[int]:
    """Device address of a tensor (checked: device, contiguity, dtype, size) or int."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and x.dtype not in dtype:
        raise TypeError(f"{name}: dtype {x.dtype} not in {dtype}")
    if count is not None and x.numel() != count:
        raise ValueError(f"{name}: {x.numel()} elements, the dimensions need {count}")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _in_types(d: Dims):
    import torch
    return (torch.bfloat16,) if d.in_dtype == IN_BF16 else (torch.float32,)


def _f32():
    import torch
    return (torch.float32,)


def _sk_types(d: Dims, f32):
    """Dtype set of the sketch (None when only raw addresses are passed)."""
    if f32 is None:
        return None
    import torch
    return (torch.bfloat16,) if d.sketch_dtype == SKETCH_BF16 else (torch.float32,)


def _check(status: int):
    if status != 0:
        raise SSMError(status, _lib.ssm_last_error().decode())


def _types(d: Dims, args):
    """Dtype sets only when tensors are passed (raw ints skip the torch import)."""
    if all(a is None or isinstance(a, int) for a in args):
        return None, None
    return _in_types(d), _f32()


def _all_raw(args) -> bool:
    return all(a is None or isinstance(a, int) for a in args)


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI, without the ssm_ prefix)
# ----------------------------------------------------------------------------
def buffer_append(d: Dims, k_t, v_t, decay_t, beta_t, k_buf, v_buf, decay_buf, beta_buf,
                  slot: int, stream=None) -> None:
    if isinstance(stream, int) and _all_raw((k_t, v_t, decay_t, beta_t, k_buf, v_buf, decay_buf,
                                             beta_buf)):
        return _check(_lib.ssm_buffer_append(ctypes.byref(d), k_t, v_t, decay_t, beta_t, k_buf,
                                             v_buf, decay_buf, beta_buf, slot, stream))
    tin, f32 = _types(d, (k_t, v_t, decay_t, beta_t, k_buf, v_buf, decay_buf, beta_buf))
    n = numel(d)
    _check(_lib.ssm_buffer_append(
        ctypes.byref(d), _addr(k_t, "k_t", tin, n["k_t"]), _addr(v_t, "v_t", tin, n["v_t"]),
        _addr(decay_t, "decay_t", f32, n["decay_t"]), _addr(beta_t, "beta_t", f32, n["beta_t"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]), _addr(beta_buf, "beta_buf", f32, n["beta_buf"]),
        int(slot), _stream(stream)))


def window_update_refresh(d: Dims, state, sketch, basis, k_buf, v_buf, decay_buf, beta_buf,
                          n_tokens: int, stream=None) -> None:
    if isinstance(stream, int) and _all_raw((state, sketch, basis, k_buf, v_buf, decay_buf,
                                             beta_buf)):
        return _check(_lib.ssm_window_update_refresh(ctypes.byref(d), state, sketch, basis, k_buf,
                                                     v_buf, decay_buf, beta_buf, n_tokens, stream))
    tin, f32 = _types(d, (state, sketch, basis, k_buf, v_buf, decay_buf, beta_buf))
    n = numel(d)
    _check(_lib.ssm_window_update_refresh(
        ctypes.byref(d), _addr(state, "state", f32, n["state"]), _addr(sketch, "sketch", _sk_types(d, f32), n["sketch"]),
        _addr(basis, "basis", f32, n["basis"]), _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]), _addr(beta_buf, "beta_buf", f32, n["beta_buf"]),
        int(n_tokens), _stream(stream)))


def sketch_decode_step(d: Dims, sketch, basis, q, k_buf, v_buf, decay_buf, beta_buf, tau: int,
                       y, *, k_t=None, v_t=None, decay_t=None, beta_t=None, stream=None) -> None:
    if isinstance(stream, int) and _all_raw((sketch, basis, q, k_buf, v_buf, decay_buf, beta_buf,
                                             y, k_t, v_t, decay_t, beta_t)):
        return _check(_lib.ssm_sketch_decode_step(ctypes.byref(d), sketch, basis, q, k_t, v_t,
                                                  decay_t, beta_t, k_buf, v_buf, decay_buf,
                                                  beta_buf, tau, y, stream))
    tin, f32 = _types(d, (sketch, basis, q, k_buf, v_buf, decay_buf, beta_buf, y, k_t, v_t))
    n = numel(d)
    _check(_lib.ssm_sketch_decode_step(
        ctypes.byref(d), _addr(sketch, "sketch", _sk_types(d, f32), n["sketch"]), _addr(basis, "basis", f32, n["basis"]),
        _addr(q, "q", tin, n["q"]), _addr(k_t, "k_t", tin, n["k_t"]), _addr(v_t, "v_t", tin, n["v_t"]),
        _addr(decay_t, "decay_t", f32, n["decay_t"]), _addr(beta_t, "beta_t", f32, n["beta_t"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]), _addr(beta_buf, "beta_buf", f32, n["beta_buf"]),
        int(tau), _addr(y, "y", f32, n["y"]), _stream(stream)))


def full_read_decode_step(d: Dims, state, q, k_buf, v_buf, decay_buf, beta_buf, tau: int, y, *,
                          k_t=None, v_t=None, decay_t=None, beta_t=None, stream=None) -> None:
    if isinstance(stream, int) and _all_raw((state, q, k_buf, v_buf, decay_buf, beta_buf, y, k_t,
                                             v_t, decay_t, beta_t)):
        return _check(_lib.ssm_full_read_decode_step(ctypes.byref(d), state, q, k_t, v_t, decay_t,
                                                     beta_t, k_buf, v_buf, decay_buf, beta_buf,
                                                     tau, y, stream))
    tin, f32 = _types(d, (state, q, k_buf, v_buf, decay_buf, beta_buf, y, k_t, v_t))
    n = numel(d)
    _check(_lib.ssm_full_read_decode_step(
        ctypes.byref(d), _addr(state, "state", f32, n["state"]), _addr(q, "q", tin, n["q"]),
        _addr(k_t, "k_t", tin, n["k_t"]), _addr(v_t, "v_t", tin, n["v_t"]),
        _addr(decay_t, "decay_t", f32, n["decay_t"]), _addr(beta_t, "beta_t", f32, n["beta_t"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]), _addr(beta_buf, "beta_buf", f32, n["beta_buf"]),
        int(tau), _addr(y, "y", f32, n["y"]), _stream(stream)))


def recurrent_decode_step(d: Dims, state, q, k_t, v_t, decay_t, beta_t, y, stream=None) -> None:
    if isinstance(stream, int) and _all_raw((state, q, k_t, v_t, decay_t, beta_t, y)):
        return _check(_lib.ssm_recurrent_decode_step(ctypes.byref(d), state, q, k_t, v_t, decay_t,
                                                     beta_t, y, stream))
    tin, f32 = _types(d, (state, q, k_t, v_t, decay_t, beta_t, y))
    n = numel(d)
    _check(_lib.ssm_recurrent_decode_step(
        ctypes.byref(d), _addr(state, "state", f32, n["state"]), _addr(q, "q", tin, n["q"]),
        _addr(k_t, "k_t", tin, n["k_t"]), _addr(v_t, "v_t", tin, n["v_t"]),
        _addr(decay_t, "decay_t", f32, n["decay_t"]), _addr(beta_t, "beta_t", f32, n["beta_t"]),
        _addr(y, "y", f32, n["y"]), _stream(stream)))


def fit_basis(d: Dims, samples, n_samples: int, basis, stream=None) -> None:
    """ssm_fit_basis: per head, the d.rank leading eigenvectors of the samples' uncentred
    second moment as orthonormal rows of basis. samples [H][n_samples][d_k] (d.in_dtype),
    basis [H][rank][d_k] fp32."""
    if isinstance(stream, int) and _all_raw((samples, basis)):
        return _check(_lib.ssm_fit_basis(ctypes.byref(d), samples, int(n_samples), basis, stream))
    tin, f32 = _types(d, (samples, basis))
    _check(_lib.ssm_fit_basis(
        ctypes.byref(d), _addr(samples, "samples", tin, d.heads * int(n_samples) * d.d_k),
        int(n_samples), _addr(basis, "basis", f32, d.heads * d.rank * d.d_k), _stream(stream)))


def stream_probe(buf, n_tiles: int, shape: int, stream=None) -> None:
    """ssm_stream_probe (a measurement aid): stream buf, n_tiles 64 KB fp32 tiles, in place
    in access shape 0 (the window update's order) or 1 (flat runs of two tiles)."""
    ptr = buf if isinstance(buf, int) else _addr(buf, "buf", _f32(), int(n_tiles) * 16384)
    _check(_lib.ssm_stream_probe(ptr, int(n_tiles), int(shape), _stream(stream)))


# ----------------------------------------------------------------------------
# heterogeneous per-head sketch ranks
# ----------------------------------------------------------------------------
def rank_offsets(ranks) -> "ctypes.Array":
    """Host int32 prefix offsets (H + 1 values) for per-head ranks."""
    off = [0]
    for r in ranks:
        off.append(off[-1] + int(r))
    return (ctypes.c_int32 * len(off))(*off)


def _ranked_numel(d: Dims, offsets) -> dict:
    n = numel(d)
    R = int(offsets[d.heads]) if len(offsets) > d.heads else 0
    n["sketch"] = d.batch * R * d.d_v
    n["basis"] = R * d.d_k
    return n


def _offsets_arg(d: Dims, offsets):
    if not isinstance(offsets, ctypes.Array):
        offsets = rank_offsets(offsets) if len(offsets) == d.heads else \
            (ctypes.c_int32 * len(offsets))(*[int(x) for x in offsets])
    if len(offsets) != d.heads + 1:
        raise ValueError(f"rank_offsets: {len(offsets)} entries, need heads + 1 = {d.heads + 1}")
    return offsets


def window_update_refresh_ranked(d: Dims, offsets, state, sketch, basis, k_buf, v_buf,
                                 decay_buf, beta_buf, n_tokens: int, stream=None) -> None:
    """ssm_window_update_refresh_ranked. `offsets`: H + 1 prefix offsets, or H per-head ranks."""
    off = _offsets_arg(d, offsets)
    if isinstance(stream, int) and _all_raw((state, sketch, basis, k_buf, v_buf, decay_buf,
                                             beta_buf)):
        return _check(_lib.ssm_window_update_refresh_ranked(
            ctypes.byref(d), off, state, sketch, basis, k_buf, v_buf, decay_buf, beta_buf,
            n_tokens, stream))
    tin, f32 = _types(d, (state, sketch, basis, k_buf, v_buf, decay_buf, beta_buf))
    n = _ranked_numel(d, off)
    _check(_lib.ssm_window_update_refresh_ranked(
        ctypes.byref(d), off, _addr(state, "state", f32, n["state"]),
        _addr(sketch, "sketch", _sk_types(d, f32), n["sketch"]), _addr(basis, "basis", f32, n["basis"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]),
        _addr(beta_buf, "beta_buf", f32, n["beta_buf"]), int(n_tokens), _stream(stream)))


def sketch_decode_step_ranked(d: Dims, offsets, sketch, basis, q, k_buf, v_buf, decay_buf,
                              beta_buf, tau: int, y, *, k_t=None, v_t=None, decay_t=None,
                              beta_t=None, stream=None) -> None:
    """ssm_sketch_decode_step_ranked. `offsets`: H + 1 prefix offsets, or H per-head ranks."""
    off = _offsets_arg(d, offsets)
    if isinstance(stream, int) and _all_raw((sketch, basis, q, k_buf, v_buf, decay_buf, beta_buf,
                                             y, k_t, v_t, decay_t, beta_t)):
        return _check(_lib.ssm_sketch_decode_step_ranked(
            ctypes.byref(d), off, sketch, basis, q, k_t, v_t, decay_t, beta_t, k_buf, v_buf,
            decay_buf, beta_buf, tau, y, stream))
    tin, f32 = _types(d, (sketch, basis, q, k_buf, v_buf, decay_buf, beta_buf, y, k_t, v_t))
    n = _ranked_numel(d, off)
    _check(_lib.ssm_sketch_decode_step_ranked(
        ctypes.byref(d), off, _addr(sketch, "sketch", _sk_types(d, f32), n["sketch"]),
        _addr(basis, "basis", f32, n["basis"]), _addr(q, "q", tin, n["q"]),
        _addr(k_t, "k_t", tin, n["k_t"]), _addr(v_t, "v_t", tin, n["v_t"]),
        _addr(decay_t, "decay_t", f32, n["decay_t"]), _addr(beta_t, "beta_t", f32, n["beta_t"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]),
        _addr(beta_buf, "beta_buf", f32, n["beta_buf"]), int(tau), _addr(y, "y", f32, n["y"]),
        _stream(stream)))


# ----------------------------------------------------------------------------
# variable-length batches over a pool of slots
# ----------------------------------------------------------------------------
def _pool_numel(d: Dims, num_slots: int) -> dict:
    n = numel(d)
    p = numel(Dims(d.rule, d.in_dtype, num_slots, d.heads, d.d_k, d.d_v, d.window, d.rank))
    for key in ("state", "sketch", "k_buf", "v_buf", "decay_buf", "beta_buf"):
        n[key] = p[key]
    n["rows"] = d.batch
    return n


def _i32():
    import torch
    return (torch.int32,)


def window_update_refresh_varlen(d: Dims, num_slots: int, slot, n_tokens, state, sketch, basis,
                                 k_buf, v_buf, decay_buf, beta_buf, stream=None) -> None:
    """ssm_window_update_refresh_varlen: per-row token counts (device int32 [batch]) and an
    optional slot map (device int32 [batch]) into a pool of num_slots persistent slots."""
    args = (slot, n_tokens, state, sketch, basis, k_buf, v_buf, decay_buf, beta_buf)
    if isinstance(stream, int) and _all_raw(args):
        return _check(_lib.ssm_window_update_refresh_varlen(ctypes.byref(d), int(num_slots), *args,
                                                            stream))
    tin, f32 = _types(d, args)
    i32 = None if tin is None else _i32()
    n = _pool_numel(d, num_slots)
    _check(_lib.ssm_window_update_refresh_varlen(
        ctypes.byref(d), int(num_slots), _addr(slot, "slot", i32, n["rows"]),
        _addr(n_tokens, "n_tokens", i32, n["rows"]), _addr(state, "state", f32, n["state"]),
        _addr(sketch, "sketch", _sk_types(d, f32), n["sketch"]), _addr(basis, "basis", f32, n["basis"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]),
        _addr(beta_buf, "beta_buf", f32, n["beta_buf"]), _stream(stream)))


def sketch_decode_step_varlen(d: Dims, num_slots: int, slot, tau, sketch, basis, q, k_buf, v_buf,
                              decay_buf, beta_buf, y, *, k_t=None, v_t=None, decay_t=None,
                              beta_t=None, stream=None) -> None:
    """ssm_sketch_decode_step_varlen: per-row window positions tau (device int32 [batch])."""
    args = (slot, tau, sketch, basis, q, k_t, v_t, decay_t, beta_t, k_buf, v_buf, decay_buf,
            beta_buf, y)
    if isinstance(stream, int) and _all_raw(args):
        return _check(_lib.ssm_sketch_decode_step_varlen(ctypes.byref(d), int(num_slots), *args,
                                                         stream))
    tin, f32 = _types(d, args)
    i32 = None if tin is None else _i32()
    n = _pool_numel(d, num_slots)
    _check(_lib.ssm_sketch_decode_step_varlen(
        ctypes.byref(d), int(num_slots), _addr(slot, "slot", i32, n["rows"]),
        _addr(tau, "tau", i32, n["rows"]), _addr(sketch, "sketch", _sk_types(d, f32), n["sketch"]),
        _addr(basis, "basis", f32, n["basis"]), _addr(q, "q", tin, n["q"]),
        _addr(k_t, "k_t", tin, n["k_t"]), _addr(v_t, "v_t", tin, n["v_t"]),
        _addr(decay_t, "decay_t", f32, n["decay_t"]), _addr(beta_t, "beta_t", f32, n["beta_t"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]),
        _addr(beta_buf, "beta_buf", f32, n["beta_buf"]), _addr(y, "y", f32, n["y"]),
        _stream(stream)))


def decode_step_varlen(d: Dims, num_slots: int, slot, tau, parity, n_update: int, update_rows,
                       state, sketch0, sketch1, basis, q, k_t, v_t, decay_t, beta_t, k_buf,
                       v_buf, decay_buf, beta_buf, y, stream=None) -> None:
    """ssm_decode_step_varlen: one serving step in one launch. Every row reads y at its own
    window position tau (device int32 [batch]) from sketch0 or sketch1 (parity, device int32
    [batch]) with the current token appended; the n_update rows listed in update_rows (device
    int32) whose window fills (tau == W) also apply the window to the state and store the
    refreshed sketch in the other buffer."""
    args = (slot, tau, parity, update_rows, state, sketch0, sketch1, basis, q, k_t, v_t, decay_t,
            beta_t, k_buf, v_buf, decay_buf, beta_buf, y)
    if isinstance(stream, int) and _all_raw(args):
        return _check(_lib.ssm_decode_step_varlen(
            ctypes.byref(d), int(num_slots), slot, tau, parity, int(n_update), update_rows, state,
            sketch0, sketch1, basis, q, k_t, v_t, decay_t, beta_t, k_buf, v_buf, decay_buf,
            beta_buf, y, stream))
    tin, f32 = _types(d, args)
    i32 = None if tin is None else _i32()
    n = _pool_numel(d, num_slots)
    sk = _sk_types(d, f32)
    _check(_lib.ssm_decode_step_varlen(
        ctypes.byref(d), int(num_slots), _addr(slot, "slot", i32, n["rows"]),
        _addr(tau, "tau", i32, n["rows"]), _addr(parity, "parity", i32, n["rows"]),
        int(n_update), _addr(update_rows, "update_rows", i32, int(n_update) if n_update else None),
        _addr(state, "state", f32, n["state"]), _addr(sketch0, "sketch0", sk, n["sketch"]),
        _addr(sketch1, "sketch1", sk, n["sketch"]), _addr(basis, "basis", f32, n["basis"]),
        _addr(q, "q", tin, n["q"]), _addr(k_t, "k_t", tin, n["k_t"]),
        _addr(v_t, "v_t", tin, n["v_t"]), _addr(decay_t, "decay_t", f32, n["decay_t"]),
        _addr(beta_t, "beta_t", f32, n["beta_t"]), _addr(k_buf, "k_buf", tin, n["k_buf"]),
        _addr(v_buf, "v_buf", tin, n["v_buf"]), _addr(decay_buf, "decay_buf", f32, n["decay_buf"]),
        _addr(beta_buf, "beta_buf", f32, n["beta_buf"]), _addr(y, "y", f32, n["y"]),
        _stream(stream)))


def window_update_refresh_ls(d: Dims, state, sketch_q, read_map, basis, k_buf, v_buf, decay_buf,
                             beta_buf, n_tokens: int, stream=None) -> None:
    """ssm_window_update_refresh_ls: the window update, then the least-squares sketch
    (orthonormal sketch rows sketch_q [N][H][r][d_v] and read_map [N][H][r][d_k])."""
    args = (state, sketch_q, read_map, basis, k_buf, v_buf, decay_buf, beta_buf)
    if isinstance(stream, int) and _all_raw(args):
        return _check(_lib.ssm_window_update_refresh_ls(ctypes.byref(d), *args, n_tokens, stream))
    tin, f32 = _types(d, args)
    n = numel(d)
    _check(_lib.ssm_window_update_refresh_ls(
        ctypes.byref(d), _addr(state, "state", f32, n["state"]),
        _addr(sketch_q, "sketch_q", f32, n["sketch"]),
        _addr(read_map, "read_map", f32, n["read_map"]), _addr(basis, "basis", f32, n["basis"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]),
        _addr(beta_buf, "beta_buf", f32, n["beta_buf"]), int(n_tokens), _stream(stream)))


def sketch_decode_step_ls(d: Dims, sketch_q, read_map, q, k_buf, v_buf, decay_buf, beta_buf,
                          tau: int, y, *, k_t=None, v_t=None, decay_t=None, beta_t=None,
                          stream=None) -> None:
    """ssm_sketch_decode_step_ls: y = sketch_q^T (read_map q~) + R^T q."""
    args = (sketch_q, read_map, q, k_buf, v_buf, decay_buf, beta_buf, y, k_t, v_t, decay_t,
            beta_t)
    if isinstance(stream, int) and _all_raw(args):
        return _check(_lib.ssm_sketch_decode_step_ls(ctypes.byref(d), sketch_q, read_map, q, k_t,
                                                     v_t, decay_t, beta_t, k_buf, v_buf,
                                                     decay_buf, beta_buf, tau, y, stream))
    tin, f32 = _types(d, args)
    n = numel(d)
    _check(_lib.ssm_sketch_decode_step_ls(
        ctypes.byref(d), _addr(sketch_q, "sketch_q", f32, n["sketch"]),
        _addr(read_map, "read_map", f32, n["read_map"]), _addr(q, "q", tin, n["q"]),
        _addr(k_t, "k_t", tin, n["k_t"]), _addr(v_t, "v_t", tin, n["v_t"]),
        _addr(decay_t, "decay_t", f32, n["decay_t"]), _addr(beta_t, "beta_t", f32, n["beta_t"]),
        _addr(k_buf, "k_buf", tin, n["k_buf"]), _addr(v_buf, "v_buf", tin, n["v_buf"]),
        _addr(decay_buf, "decay_buf", f32, n["decay_buf"]),
        _addr(beta_buf, "beta_buf", f32, n["beta_buf"]), int(tau), _addr(y, "y", f32, n["y"]),
        _stream(stream)))
