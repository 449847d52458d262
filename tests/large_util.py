"""Host-side windows of counter-based inputs (input_dependent_short_amd.inputs.
counter_values) and the oracle evaluated on them: for tensors that exist only on
the GPU, the oracle sees a token window (or a channel slice) rebuilt on the host.

A token window [wlo, whi) around the checked rows [lo, hi) reaches W-1 tokens
to each side, so every tap of those rows lies inside it.  The window is passed
to the oracle as a batch of its own whose sequences start at the window start
and at every true sequence start inside it; the checked rows then see exactly
the taps they see in the whole tensor.  Channel slices serve the sums over all
tokens (dU, dc), which involve each channel on its own.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from input_dependent_short_amd import inputs
from input_dependent_short_amd.inputs import to_f64


def rows_of(seed: int, std: float, dtype: str, tail: tuple, lo: int, hi: int) -> np.ndarray:
    """Rows [lo, hi) of an (N, *tail) counter tensor, as exact doubles."""
    per = int(np.prod(tail))
    idx = torch.arange(lo * per, hi * per, dtype=torch.int64)
    return to_f64(inputs.counter_values(seed, idx, std, dtype)).reshape(hi - lo, *tail)


def channels_of(seed: int, std: float, dtype: str, N: int, D: int, c0: int, c1: int) -> np.ndarray:
    """Channels [c0, c1) of every token of an (N, D) counter tensor."""
    idx = torch.arange(N, dtype=torch.int64)[:, None] * D + torch.arange(c0, c1, dtype=torch.int64)[None, :]
    return to_f64(inputs.counter_values(seed, idx.reshape(-1), std, dtype)).reshape(N, c1 - c0)


def window_cu(T: int, wlo: int, whi: int, cu=None) -> np.ndarray:
    """Sequence offsets of the window [wlo, whi) of a batch of rows of T tokens
    (each row one sequence), or of packed sequences with offsets ``cu``."""
    inside = range((wlo // T + 1) * T, whi, T) if cu is None else [int(c) for c in cu if wlo < c < whi]
    starts = {0, whi - wlo} | {s - wlo for s in inside}
    return np.array(sorted(starts), dtype=np.int32)


def window(N: int, W: int, lo: int, hi: int) -> tuple[int, int]:
    return max(0, lo - (W - 1)), min(N, hi + (W - 1))


def headwise_rows(seeds: dict, N: int, T: int, D: int, G: int, W: int, lo: int, hi: int, residual: bool,
                  dtype: str, cu=None):
    """Oracle (y, dx, dw) of rows [lo, hi) of a head-wise layer on counter inputs."""
    wlo, whi = window(N, W, lo, hi)
    L = whi - wlo
    x = rows_of(seeds["x"], 1.0, dtype, (D,), wlo, whi).reshape(1, L, D)
    w = rows_of(seeds["w"], 1.0 / np.sqrt(W), dtype, (G, W), wlo, whi).reshape(1, L, G, W)
    dy = rows_of(seeds["dy"], 1.0, dtype, (D,), wlo, whi).reshape(1, L, D)
    cu, rows = window_cu(T, wlo, whi, cu), (lo - wlo, hi - wlo)
    y = oracle.headwise_fwd(x, w, cu_seqlens=cu, residual=residual, rows=rows)
    dx, dw = oracle.headwise_bwd(x, w, dy, cu_seqlens=cu, residual=residual, rows=rows)
    return y, dx, dw


def lowrank_U(seeds: dict, R: int, D: int, W: int, dtype: str) -> np.ndarray:
    return rows_of(seeds["U"], 1.0 / np.sqrt(R * W), dtype, (D * W,), 0, R)


def lowrank_rows(seeds: dict, N: int, T: int, D: int, R: int, W: int, lo: int, hi: int, residual: bool,
                 dtype: str, cu=None):
    """Oracle (y, dx, dz) of rows [lo, hi) of a low-rank layer on counter inputs."""
    wlo, whi = window(N, W, lo, hi)
    L = whi - wlo
    x = rows_of(seeds["x"], 1.0, dtype, (D,), wlo, whi).reshape(1, L, D)
    z = rows_of(seeds["z"], 1.0, dtype, (R,), wlo, whi).reshape(1, L, R)
    dy = rows_of(seeds["dy"], 1.0, dtype, (D,), wlo, whi).reshape(1, L, D)
    U = lowrank_U(seeds, R, D, W, dtype)
    cu, rows = window_cu(T, wlo, whi, cu), (lo - wlo, hi - wlo)
    y = oracle.lowrank_fwd(x, z, U, W, cu_seqlens=cu, residual=residual, rows=rows)
    dx, dz, _ = oracle.lowrank_bwd(x, z, U, dy, W, cu_seqlens=cu, residual=residual, rows=rows, channels=(0, 0))
    return y, dx, dz


def lowrank_dU(seeds: dict, B: int, T: int, D: int, R: int, W: int, c0: int, c1: int, dtype: str,
               cu=None) -> np.ndarray:
    """Oracle dU of channels [c0, c1), (R, (c1-c0)*W), summed over every token."""
    N, dc = B * T, c1 - c0
    x = channels_of(seeds["x"], 1.0, dtype, N, D, c0, c1).reshape(B, T, dc)
    dy = channels_of(seeds["dy"], 1.0, dtype, N, D, c0, c1).reshape(B, T, dc)
    z = rows_of(seeds["z"], 1.0, dtype, (R,), 0, N).reshape(B, T, R)
    U = lowrank_U(seeds, R, D, W, dtype).reshape(R, D, W)[:, c0:c1].reshape(R, dc * W)
    return oracle.lowrank_bwd(x, z, U, dy, W, cu_seqlens=cu, rows=(0, 0), channels=(0, dc))[2]


def static_c(seeds: dict, D: int, W: int, dtype: str) -> np.ndarray:
    return rows_of(seeds["c"], 1.0 / np.sqrt(W), dtype, (W,), 0, D)


def static_rows(seeds: dict, N: int, T: int, D: int, W: int, lo: int, hi: int, residual: bool, dtype: str,
                cu=None):
    """Oracle (y, dx) of rows [lo, hi) of the static layer on counter inputs."""
    wlo, whi = window(N, W, lo, hi)
    L = whi - wlo
    x = rows_of(seeds["x"], 1.0, dtype, (D,), wlo, whi).reshape(1, L, D)
    dy = rows_of(seeds["dy"], 1.0, dtype, (D,), wlo, whi).reshape(1, L, D)
    c = static_c(seeds, D, W, dtype)
    cu, rows = window_cu(T, wlo, whi, cu), (lo - wlo, hi - wlo)
    y = oracle.static_fwd(x, c, cu_seqlens=cu, residual=residual, rows=rows)
    dx, _ = oracle.static_bwd(x, c, dy, cu_seqlens=cu, residual=residual, rows=rows)
    return y, dx


def static_dc(seeds: dict, B: int, T: int, D: int, W: int, c0: int, c1: int, dtype: str) -> np.ndarray:
    """Oracle dc of channels [c0, c1), summed over every token."""
    N, dc = B * T, c1 - c0
    x = channels_of(seeds["x"], 1.0, dtype, N, D, c0, c1).reshape(B, T, dc)
    dy = channels_of(seeds["dy"], 1.0, dtype, N, D, c0, c1).reshape(B, T, dc)
    c = static_c(seeds, D, W, dtype)[c0:c1]
    return oracle.static_bwd(x, c, dy, rows=(0, 0))[1]
