"""Independent brute-force forms of the dynamic short convolution (numpy, fp64).

Test helper, separate from the oracle: the convolution of one channel is
written as a dense N x N lower-banded matrix A with A[t, t-k] = filter_t[k]
for t-k inside t's segment, so that y = rho*x + A x and dx = rho*g + A^T g.
Low-rank filters are materialised with einsum.
"""
from __future__ import annotations

import numpy as np


def seg_starts(B: int, T: int, cu_seqlens=None) -> np.ndarray:
    N = B * T
    if cu_seqlens is None:
        return (np.arange(N) // T) * T
    s = np.empty(N, dtype=np.int64)
    cu = list(cu_seqlens)
    for i in range(len(cu) - 1):
        s[cu[i]:cu[i + 1]] = cu[i]
    return s


def band_matrix(filt: np.ndarray, seg: np.ndarray) -> np.ndarray:
    """filt (N, W) taps of one channel for every token -> dense (N, N) matrix."""
    N, W = filt.shape
    A = np.zeros((N, N))
    for t in range(N):
        for k in range(W):
            s = t - k
            if s >= seg[t]:
                A[t, s] = filt[t, k]
    return A


def perchannel_filters_headwise(w: np.ndarray, D: int) -> np.ndarray:
    """w (B,T,G,W) -> per-channel filters (N, D, W) by repeating each group H times."""
    B, T, G, W = w.shape
    return np.repeat(w.reshape(B * T, G, W), D // G, axis=1)


def perchannel_filters_lowrank(z: np.ndarray, U: np.ndarray, W: int) -> np.ndarray:
    B, T, R = z.shape
    D = U.shape[1] // W
    return np.einsum("nr,rdk->ndk", z.reshape(B * T, R), U.reshape(R, D, W))


def conv_fwd(x: np.ndarray, filt_pc: np.ndarray, seg: np.ndarray, residual: bool) -> np.ndarray:
    B, T, D = x.shape
    xf = x.reshape(B * T, D)
    y = np.zeros_like(xf)
    for d in range(D):
        y[:, d] = band_matrix(filt_pc[:, d, :], seg) @ xf[:, d]
    if residual:
        y += xf
    return y.reshape(B, T, D)


def conv_dx(g: np.ndarray, filt_pc: np.ndarray, seg: np.ndarray, residual: bool) -> np.ndarray:
    B, T, D = g.shape
    gf = g.reshape(B * T, D)
    dx = np.zeros_like(gf)
    for d in range(D):
        dx[:, d] = band_matrix(filt_pc[:, d, :], seg).T @ gf[:, d]
    if residual:
        dx += gf
    return dx.reshape(B, T, D)
