"""Seeded synthetic inputs for the SketchSSM windowed decode layer.

This module only draws numbers. It holds none of the method's arithmetic: no
recurrence, no decomposition, no sketch. Both the CPU oracle (through the
tests) and the HIP library (through the tests and the benchmark) take their
inputs from here, so the two sides see bit-identical values.

The SketchSSM pages (arXiv 2609.33051, abstract) evaluate on Mamba-2, Gated
DeltaNet and KDA based models; no weights or datasets are available, so these
tensors stand in for one linear-attention layer's decode inputs with the
shapes, dtypes and gate distributions of the five workloads below. The state
size does not depend on context length, so a layer's decode cost depends only
on these shapes and the batch.

Conventions
-----------
* ``N(mu, s)`` is read as mean ``mu`` and standard deviation ``s``.
* Seeds: ``np.random.default_rng([0x5EED, cfg_id, stream, index])`` with the
  streams below; per-step inputs use ``index = step``, the initial state uses
  ``index = sequence``.
* bf16 values are produced from fp32 by round-to-nearest-even and are carried
  as ``uint16`` bit patterns; :func:`widen` turns them back into exact floats.
* Layouts (row-major): q, k ``[N][H][d_k]``; v ``[N][H][d_v]``; decay
  ``[N][H]`` (scalar gate) or ``[N][H][d_k]`` (per-channel gate); beta
  ``[N][H]``; initial state ``[N][H][d_k][d_v]``; basis ``[H][r][d_k]`` (row m
  is basis vector b_m, orthonormal rows).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED = 0x5EED

# RNG streams
STREAM_S0 = 0
STREAM_BASIS = 1
STREAM_PCA = 2
STREAM_Q = 3
STREAM_K = 4
STREAM_V = 5
STREAM_GATES = 6
STREAM_A = 7

RULES = ("mamba2", "gdn", "kda")


@dataclasses.dataclass(frozen=True)
class Config:
    """One decode-layer workload."""

    name: str
    cfg_id: int
    rule: str            # "mamba2" | "gdn" | "kda"
    in_dtype: str        # "bf16" | "f32"  (q, k, v)
    batch: int
    heads: int
    d_k: int
    d_v: int
    window: int
    rank: int
    steps: int
    qkv_recipe: str      # "scaled_normal" | "l2norm_qk"
    gate_recipe: str     # "uniform" | "mamba2_dt" | "uniform_channel"
    gate_lo: float = 0.90
    gate_hi: float = 0.999
    basis_recipe: str = "qr"   # "qr" | "pca"
    description: str = ""

    @property
    def units(self) -> int:
        return self.batch * self.heads

    @property
    def per_channel_decay(self) -> bool:
        return self.rule == "kda"

    @property
    def has_beta(self) -> bool:
        return self.rule in ("gdn", "kda")

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


C1 = Config(
    name="c1", cfg_id=1, rule="mamba2", in_dtype="f32", batch=2, heads=4,
    d_k=16, d_v=32, window=4, rank=4, steps=16, qkv_recipe="scaled_normal",
    gate_recipe="uniform", gate_lo=0.90, gate_hi=0.999, basis_recipe="qr",
    description="tiny Mamba-2-style layer, fp32 inputs, N=2 H=4 d_k=16 d_v=32 W=4 r=4 T=16",
)
C2 = Config(
    name="c2", cfg_id=2, rule="mamba2", in_dtype="bf16", batch=256, heads=80,
    d_k=128, d_v=64, window=8, rank=8, steps=64, qkv_recipe="scaled_normal",
    gate_recipe="mamba2_dt", basis_recipe="pca",
    description="Mamba-2 decode layer, N=256 H=80 d_state=128 headdim=64 W=8 r=8 T=64",
)
C3 = Config(
    name="c3", cfg_id=3, rule="gdn", in_dtype="bf16", batch=256, heads=32,
    d_k=128, d_v=128, window=8, rank=8, steps=64, qkv_recipe="l2norm_qk",
    gate_recipe="uniform", gate_lo=0.90, gate_hi=0.999, basis_recipe="qr",
    description="Gated DeltaNet decode layer, N=256 H=32 d_k=d_v=128 W=8 r=8 T=64",
)
C4 = Config(
    name="c4", cfg_id=4, rule="kda", in_dtype="bf16", batch=512, heads=32,
    d_k=128, d_v=128, window=8, rank=8, steps=64, qkv_recipe="l2norm_qk",
    gate_recipe="uniform_channel", gate_lo=0.85, gate_hi=0.999, basis_recipe="qr",
    description="KDA decode layer, N=512 H=32 d_k=d_v=128 W=8 r=8 T=64",
)
# The sweep on the Gated DeltaNet layer: one token stream, 12 (r, W) points.
C5_RANKS = (4, 8, 16, 32)
C5_WINDOWS = (4, 8, 16)
C5_BASE = C3.with_(name="c5", cfg_id=5, batch=1024, steps=128,
                   description="Gated DeltaNet sweep, N=1024 H=32 d_k=d_v=128 T=128")


def c5(rank: int, window: int) -> Config:
    if rank not in C5_RANKS or window not in C5_WINDOWS:
        raise ValueError(f"sweep point r={rank} W={window} is not on the grid")
    return C5_BASE.with_(name=f"c5_r{rank}_w{window}", rank=rank, window=window,
                         description=f"{C5_BASE.description}, r={rank} W={window}")


CONFIGS = {c.name: c for c in (C1, C2, C3, C4)}
for _r in C5_RANKS:
    for _w in C5_WINDOWS:
        CONFIGS[f"c5_r{_r}_w{_w}"] = c5(_r, _w)


def get(name: str) -> Config:
    return CONFIGS[name]


def _rng(cfg: Config, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED, cfg.cfg_id, stream, index])


# --------------------------------------------------------------------------
# bf16 plumbing
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def widen(x: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bf16 bits (uint16) or float arrays -> exact values in ``dtype``."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype)
    return x.astype(dtype)


def _pack(cfg: Config, x: np.ndarray) -> np.ndarray:
    if cfg.in_dtype == "bf16":
        return to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _l2norm(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass
class StepInputs:
    """Decode inputs of one token for every (sequence, head)."""

    q: np.ndarray                 # [N][H][d_k]  uint16 (bf16 bits) or float32
    k: np.ndarray                 # [N][H][d_k]
    v: np.ndarray                 # [N][H][d_v]
    decay: np.ndarray             # [N][H] or [N][H][d_k] float32
    beta: Optional[np.ndarray]    # [N][H] float32, None for Mamba-2


def _queries(cfg: Config, rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if cfg.qkv_recipe == "l2norm_qk":
        return _l2norm(x)
    return x / np.float32(np.sqrt(cfg.d_k))


def head_scale_A(cfg: Config) -> np.ndarray:
    """Mamba-2 per-head A ~ U(1, 16)."""
    return _rng(cfg, STREAM_A).uniform(1.0, 16.0, size=cfg.heads).astype(np.float32)


def step_inputs(cfg: Config, t: int) -> StepInputs:
    N, H, dk, dv = cfg.batch, cfg.heads, cfg.d_k, cfg.d_v
    q = _queries(cfg, _rng(cfg, STREAM_Q, t), (N, H, dk))
    k = _queries(cfg, _rng(cfg, STREAM_K, t), (N, H, dk))
    rv = _rng(cfg, STREAM_V, t)
    if cfg.qkv_recipe == "l2norm_qk":
        v = rv.standard_normal((N, H, dv), dtype=np.float32)
    else:
        v = rv.standard_normal((N, H, dv), dtype=np.float32) / np.float32(np.sqrt(dk))
    rg = _rng(cfg, STREAM_GATES, t)
    if cfg.gate_recipe == "uniform":
        decay = rg.uniform(cfg.gate_lo, cfg.gate_hi, size=(N, H)).astype(np.float32)
    elif cfg.gate_recipe == "uniform_channel":
        decay = rg.uniform(cfg.gate_lo, cfg.gate_hi, size=(N, H, dk)).astype(np.float32)
    elif cfg.gate_recipe == "mamba2_dt":
        dt = rg.normal(-3.0, 0.5, size=(N, H))
        A = head_scale_A(cfg).astype(np.float64)
        softplus = np.logaddexp(0.0, dt)
        decay = np.exp(-softplus * A[None, :]).astype(np.float32)
    else:
        raise ValueError(cfg.gate_recipe)
    beta = None
    if cfg.has_beta:
        z = rg.standard_normal((N, H))
        beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    return StepInputs(q=_pack(cfg, q), k=_pack(cfg, k), v=_pack(cfg, v),
                      decay=decay, beta=beta)


def initial_state(cfg: Config, seqs=None) -> np.ndarray:
    """S0 ~ N(0, 0.1^2), fp32 ``[len(seqs)][H][d_k][d_v]``; one RNG per sequence."""
    seqs = range(cfg.batch) if seqs is None else seqs
    out = np.empty((len(seqs), cfg.heads, cfg.d_k, cfg.d_v), dtype=np.float32)
    for i, n in enumerate(seqs):
        out[i] = _rng(cfg, STREAM_S0, int(n)).standard_normal(
            (cfg.heads, cfg.d_k, cfg.d_v), dtype=np.float32) * np.float32(0.1)
    return out


def _orthonormal_rows(x: np.ndarray, r: int) -> np.ndarray:
    """First r columns of the QR factor of x, returned as r orthonormal rows."""
    qm, _ = np.linalg.qr(x)
    return np.ascontiguousarray(qm[:, :r].T)


def basis(cfg: Config) -> np.ndarray:
    """Fixed offline basis, fp32 ``[H][r][d_k]`` with orthonormal rows.

    ``qr``: first r columns of the QR of an N(0,1) d_k x d_k matrix per head.
    ``pca``: per head, 4096 queries drawn like the decode queries (own RNG
    stream) -> uncentred second moment -> top-r eigenvectors -> QR.
    """
    H, dk, r = cfg.heads, cfg.d_k, cfg.rank
    out = np.empty((H, r, dk), dtype=np.float64)
    if cfg.basis_recipe == "qr":
        rng = _rng(cfg, STREAM_BASIS)
        for h in range(H):
            out[h] = _orthonormal_rows(rng.standard_normal((dk, dk)), r)
    elif cfg.basis_recipe == "pca":
        rng = _rng(cfg, STREAM_PCA)
        for h in range(H):
            qs = _queries(cfg, rng, (4096, dk)).astype(np.float64)
            second = qs.T @ qs / 4096.0
            w, vecs = np.linalg.eigh(second)
            top = vecs[:, np.argsort(w)[::-1][:r]]
            out[h] = _orthonormal_rows(top, r)
    else:
        raise ValueError(cfg.basis_recipe)
    return out.astype(np.float32)


def pca_samples(cfg: Config, n: int = 4096) -> np.ndarray:
    """The sampled queries of the ``pca`` basis recipe: per head, n queries drawn like
    the decode queries on the PCA stream, ``[H][n][d_k]`` in the config's input type
    (bf16 bits or fp32). :func:`basis` draws the same numbers before the bf16 rounding."""
    rng = _rng(cfg, STREAM_PCA)
    return np.stack([_pack(cfg, _queries(cfg, rng, (n, cfg.d_k))) for _ in range(cfg.heads)])


def basis_ranked(cfg: Config, ranks) -> np.ndarray:
    """Per-head ranks: head h keeps the first ranks[h] rows of its d_k-row basis
    (the same draws as basis() with r = d_k). fp32 [sum(ranks)][d_k]."""
    full = basis(cfg.with_(rank=cfg.d_k))
    return np.ascontiguousarray(np.concatenate([full[h, :int(r)] for h, r in enumerate(ranks)]))


def average_rank_8(heads: int) -> list:
    """A per-head rank pattern with mean 8 (cycles 2, 4, 8, 18)."""
    pattern = [2, 4, 8, 18]
    ranks = [pattern[h % 4] for h in range(heads)]
    if heads % 4:
        raise ValueError("heads must be a multiple of 4 for the mean-8 pattern")
    return ranks


def decay_shape(cfg: Config, lead) -> tuple:
    return tuple(lead) + ((cfg.d_k,) if cfg.per_channel_decay else ())


def units_of(cfg: Config, n_idx, h_idx):
    """Flat unit index (sequence-major, head-minor)."""
    return np.asarray(n_idx) * cfg.heads + np.asarray(h_idx)


def sample_units(cfg: Config, count: int, seed: int = 0) -> np.ndarray:
    """A sorted sample of flat unit indices that always holds the first and last unit."""
    U = cfg.units
    if count >= U:
        return np.arange(U)
    rng = np.random.default_rng([SEED, cfg.cfg_id, 99, seed])
    picks = rng.choice(np.arange(1, U - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, U - 1], picks]))
