"""The host windows of tests/large_util.py against the oracle on whole tensors
(CPU only): on a small batch of counter inputs, every window and channel slice
reproduces the rows and channels of the whole-tensor oracle exactly, so the
GPU tests beyond 4 GiB compare against the right values."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import large_util as lu
import oracle
from input_dependent_short_amd import inputs
from input_dependent_short_amd.inputs import to_f64

B, T, D, W, G, R = 3, 37, 16, 4, 4, 5
N = B * T
SEEDS = {"x": 11, "w": 12, "dy": 13, "z": 14, "U": 15, "c": 16}
WINDOWS = [(0, 5), (10, 20), (T - 2, T + 3), (2 * T - 1, 2 * T + 1), (N - 4, N)]
CU = np.array([0, 1, 9, 30, 37, 40, 41, 74, 100, N], dtype=np.int32)  # packed, crossing rows


def full(key, std, tail):
    return to_f64(inputs.counter_tensor((N, *tail), SEEDS[key], std, "bf16", "cpu"))


def test_counter_values_are_a_function_of_the_index():
    idx = torch.tensor([5, 2**31 + 3, 2**33 + 7, 5])
    v = inputs.counter_values(3, idx, 1.0, "fp32")
    assert v[0] == v[3] and len(set(v.tolist())) == 3
    assert torch.equal(inputs.counter_tensor((4, 6), 3, 1.0, "bf16", "cpu", chunk=5).reshape(-1),
                       inputs.counter_values(3, torch.arange(24), 1.0, "bf16"))
    u = inputs.counter_values(4, torch.arange(1 << 20), 0.5, "fp32").double()
    assert abs(float(u.mean())) < 0.01 and abs(float(u.var()) - 0.25) < 0.01
    assert float(u.abs().max()) <= 0.5 * np.sqrt(3.0)


def test_window_offsets():
    assert lu.window_cu(T, 10, 20).tolist() == [0, 10]
    assert lu.window_cu(T, T - 5, T + 5).tolist() == [0, 5, 10]
    assert lu.window(N, W, 0, 5) == (0, 8) and lu.window(N, W, N - 4, N) == (N - 7, N)


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("packed", [False, True])
def test_headwise_windows_match_the_whole_batch(residual, packed):
    cu = CU if packed else None
    x = full("x", 1.0, (D,)).reshape(B, T, D)
    w = full("w", 1 / np.sqrt(W), (G, W)).reshape(B, T, G, W)
    dy = full("dy", 1.0, (D,)).reshape(B, T, D)
    y = oracle.headwise_fwd(x, w, cu_seqlens=cu, residual=residual).reshape(N, D)
    dx, dw = oracle.headwise_bwd(x, w, dy, cu_seqlens=cu, residual=residual)
    dx, dw = dx.reshape(N, D), dw.reshape(N, G, W)
    for lo, hi in WINDOWS + [(5, 12), (36, 43)]:
        wy, wdx, wdw = lu.headwise_rows(SEEDS, N, T, D, G, W, lo, hi, residual, "bf16", cu)
        assert np.array_equal(wy, y[lo:hi]) and np.array_equal(wdx, dx[lo:hi]) and np.array_equal(wdw, dw[lo:hi])


@pytest.mark.parametrize("cu", [None, CU], ids=["rows", "packed"])
def test_lowrank_windows_and_channel_slices_match_the_whole_batch(cu):
    x = full("x", 1.0, (D,)).reshape(B, T, D)
    z = full("z", 1.0, (R,)).reshape(B, T, R)
    dy = full("dy", 1.0, (D,)).reshape(B, T, D)
    U = lu.lowrank_U(SEEDS, R, D, W, "bf16")
    y = oracle.lowrank_fwd(x, z, U, W, cu_seqlens=cu).reshape(N, D)
    dx, dz, dU = oracle.lowrank_bwd(x, z, U, dy, W, cu_seqlens=cu)
    dx, dz = dx.reshape(N, D), dz.reshape(N, R)
    for lo, hi in WINDOWS + [(5, 12), (36, 43)]:
        wy, wdx, wdz = lu.lowrank_rows(SEEDS, N, T, D, R, W, lo, hi, False, "bf16", cu)
        assert np.array_equal(wy, y[lo:hi]) and np.array_equal(wdx, dx[lo:hi]) and np.allclose(wdz, dz[lo:hi],
                                                                                              rtol=1e-12, atol=1e-12)
    for c0, c1 in [(0, 3), (D - 5, D)]:
        got = lu.lowrank_dU(SEEDS, B, T, D, R, W, c0, c1, "bf16", cu)
        assert np.allclose(got, dU.reshape(R, D, W)[:, c0:c1].reshape(R, -1), rtol=1e-12, atol=1e-12)


def test_static_windows_and_channel_slices_match_the_whole_batch():
    x = full("x", 1.0, (D,)).reshape(B, T, D)
    dy = full("dy", 1.0, (D,)).reshape(B, T, D)
    c = lu.static_c(SEEDS, D, W, "bf16")
    y = oracle.static_fwd(x, c, residual=True).reshape(N, D)
    dx, dc = oracle.static_bwd(x, c, dy, residual=True)
    dx = dx.reshape(N, D)
    for lo, hi in WINDOWS:
        wy, wdx = lu.static_rows(SEEDS, N, T, D, W, lo, hi, True, "bf16")
        assert np.array_equal(wy, y[lo:hi]) and np.array_equal(wdx, dx[lo:hi])
    for c0, c1 in [(0, 3), (D - 5, D)]:
        assert np.allclose(lu.static_dc(SEEDS, B, T, D, W, c0, c1, "bf16"), dc[c0:c1], rtol=1e-12, atol=1e-12)
