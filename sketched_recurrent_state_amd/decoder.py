"""Window cadence of the SketchSSM decode path for one linear-attention layer.

``WindowedDecoder`` owns the device buffers of one layer (the state, the
sketch, the W-token window buffer) and sequences the library calls:

* every decode step: the current token goes into its window slot and the
  output is read (from the sketch, or exactly from the full state);
* after the W-th token of a window: one fused update + refresh writes the
  full state once and stores the new sketch, and the window restarts.

This follows the SketchSSM pages (readsearch.ai listing of arXiv 2609.33051,
Abstract: full-state updates once per window with a sketch refresh, sketch
reads in between; agihunt.info summary, "Error control": the sketch's error
never reaches the state). Memory comes from PyTorch; all arithmetic is in the
library's kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (Dims, IN_BF16, KDA, MAMBA2, SKETCH_BF16, buffer_append, full_read_decode_step,
               rank_offsets, recurrent_decode_step, sketch_decode_step, sketch_decode_step_ls,
               sketch_decode_step_ranked, window_update_refresh, window_update_refresh_ls,
               window_update_refresh_ranked)


class WindowedDecoder:
    """One layer's decode state on one device.

    state:  fp32 [N, H, d_k, d_v] (used in place: the decoder writes it once per window)
    basis:  fp32 [H, r, d_k] with orthonormal rows, or None for the exact-read path only
    read:   "sketch" (the SketchSSM read), "full" (the exact buffered read, no
            sketch kept) or "both" (both reads of the same tokens; for checks)
    fused:  append the current token inside the read kernel instead of a
            separate buffering launch
    ranks:  optional per-head sketch ranks (H values); then basis is fp32 [sum(ranks), d_k]
            and the sketch [N, sum(ranks), d_v]
    coefficients: "projection" (c = B q~) or "least_squares" (c minimising the error of the
            window-start read; then `sketch` holds orthonormal sketch rows and `read_map`
            [N, H, r, d_k] the per-unit map q~ -> c; uniform rank and fp32 sketch only)
    The sketch is kept in dims.sketch_dtype (fp32, or bf16 rounded to nearest).
    """

    def __init__(self, dims: Dims, state: torch.Tensor, basis: Optional[torch.Tensor] = None, *,
                 read: str = "sketch", fused: bool = True, ranks=None,
                 coefficients: str = "projection"):
        if read not in ("sketch", "full", "both"):
            raise ValueError(read)
        if coefficients not in ("projection", "least_squares"):
            raise ValueError(coefficients)
        self.ls = coefficients == "least_squares"
        if self.ls and ranks is not None:
            raise ValueError("least-squares coefficients use a uniform rank")
        if read != "full" and basis is None:
            raise ValueError("a sketch read needs a basis")
        self.d = dims
        self.read = read
        self.fused = fused
        dev = state.device
        N, H, dk, dv, W, r = dims.batch, dims.heads, dims.d_k, dims.d_v, dims.window, dims.rank
        tin = torch.bfloat16 if dims.in_dtype == IN_BF16 else torch.float32
        self.state = state
        self.basis = basis
        self.offsets = rank_offsets(ranks) if ranks is not None else None
        rows = (H, r) if ranks is None else (int(self.offsets[H]),)
        sk_dtype = torch.bfloat16 if dims.sketch_dtype == SKETCH_BF16 else torch.float32
        self.sketch = (torch.empty((N,) + rows + (dv,), device=dev, dtype=sk_dtype)
                       if read != "full" else None)
        self.read_map = (torch.empty((N, H, r, dk), device=dev, dtype=torch.float32)
                         if self.ls and read != "full" else None)
        self.k_buf = torch.zeros((N, H, W, dk), device=dev, dtype=tin)
        self.v_buf = torch.zeros((N, H, W, dv), device=dev, dtype=tin)
        dshape = (N, H, W, dk) if dims.rule == KDA else (N, H, W)
        self.decay_buf = torch.zeros(dshape, device=dev, dtype=torch.float32)
        self.beta_buf = (torch.zeros((N, H, W), device=dev, dtype=torch.float32)
                         if dims.rule != MAMBA2 else None)
        self.tau = 0  # tokens already in the window buffer

    # -- library calls, uniform or per-head ranks --------------------------------
    def _update(self, n_tokens: int) -> None:
        bufs = (self.k_buf, self.v_buf, self.decay_buf, self.beta_buf)
        if n_tokens == 0:
            bufs = (None, None, None, None)
        if self.read_map is not None:
            window_update_refresh_ls(self.d, self.state, self.sketch, self.read_map, self.basis,
                                     *bufs, n_tokens)
        elif self.offsets is not None and self.sketch is not None:
            window_update_refresh_ranked(self.d, self.offsets, self.state, self.sketch, self.basis,
                                         *bufs, n_tokens)
        else:
            window_update_refresh(self.d, self.state, self.sketch,
                                  self.basis if self.sketch is not None else None, *bufs, n_tokens)

    def _sketch_read(self, q, tau, y, tok) -> None:
        bufs = (self.k_buf, self.v_buf, self.decay_buf, self.beta_buf)
        if self.read_map is not None:
            sketch_decode_step_ls(self.d, self.sketch, self.read_map, q, *bufs, tau, y, **tok)
        elif self.offsets is not None:
            sketch_decode_step_ranked(self.d, self.offsets, self.sketch, self.basis, q, *bufs, tau,
                                      y, **tok)
        else:
            sketch_decode_step(self.d, self.sketch, self.basis, q, *bufs, tau, y, **tok)

    # -- window boundary ---------------------------------------------------------
    def refresh(self) -> None:
        """Store the sketch of the current state (refresh-only pass)."""
        if self.sketch is not None:
            self._update(0)

    def flush(self) -> None:
        """Write the buffered tokens into the state now (a partial window) and refresh."""
        self._update(self.tau)
        self.tau = 0

    # -- one decode step -----------------------------------------------------------
    def step(self, q, k, v, decay, beta=None, *, y=None, y_full=None):
        """Read the output for the current token; returns y (or (y, y_full) for read="both")."""
        d = self.d
        tau = self.tau + 1
        N, H, dv = d.batch, d.heads, d.d_v
        if y is None and self.read != "full":
            y = torch.empty((N, H, dv), device=q.device, dtype=torch.float32)
        if y_full is None and self.read != "sketch":
            y_full = torch.empty((N, H, dv), device=q.device, dtype=torch.float32)
        tok = dict(k_t=k, v_t=v, decay_t=decay, beta_t=beta)
        if not self.fused:
            buffer_append(d, k, v, decay, beta, self.k_buf, self.v_buf, self.decay_buf,
                          self.beta_buf, tau - 1)
            tok = {}
        bufs = (self.k_buf, self.v_buf, self.decay_buf, self.beta_buf)
        if self.read != "full":
            self._sketch_read(q, tau, y, tok)
            tok = {}  # the token is in the buffer now
        if self.read != "sketch":
            full_read_decode_step(d, self.state, q, *bufs, tau, y_full, **tok)
        self.tau = tau
        if tau == d.window:
            self._update(tau)
            self.tau = 0
        if self.read == "both":
            return y, y_full
        return y if self.read == "sketch" else y_full


class RecurrentDecoder:
    """The per-token recurrent decode (the baseline SketchSSM is compared against):
    every step writes the token into the full state and reads y = S^T q from it."""

    def __init__(self, dims: Dims, state: torch.Tensor):
        self.d = dims
        self.state = state

    def step(self, q, k, v, decay, beta=None, *, y=None):
        d = self.d
        if y is None:
            y = torch.empty((d.batch, d.heads, d.d_v), device=q.device, dtype=torch.float32)
        recurrent_decode_step(d, self.state, q, k, v, decay, beta, y)
        return y
