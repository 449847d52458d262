"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Every ``pin_*`` function takes an ``oracle.Oracle`` (the real one, or a
variant with a planted mistake) and raises AssertionError when the oracle
disagrees with:
  - hand-worked examples of the defining formula (tests/golden),
  - the dense banded-matrix brute force (tests/bruteforce.py),
  - closed forms (impulse response, W = 1 scaling, static filters equal to
    numpy.convolve / numpy.correlate, rank-1 low-rank),
  - the adjoint identity and exact central finite differences of L = <g, y>,
  - structural identities (segment independence, locality / causality).
The formula is the one in "Dynamic Short Convolutions Improve Transformers"
(gist.science technical summary, Methodology): y_t is the sum over k < W of
w(t)_k times x_{t-k}; the pages state that it generalises the static,
causal short convolution (authors' thread on digg.com).
"""
from __future__ import annotations

import json
import os

import numpy as np

import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")
RTOL = 1e-12


def _close(a, b, tol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


def _rng(seed):
    return np.random.default_rng(seed)


def _hw_case(rng, B, T, D, W, H):
    x = rng.standard_normal((B, T, D))
    w = rng.standard_normal((B, T, D // H, W))
    g = rng.standard_normal((B, T, D))
    return x, w, g


def _lr_case(rng, B, T, D, W, R):
    x = rng.standard_normal((B, T, D))
    z = rng.standard_normal((B, T, R))
    U = rng.standard_normal((R, D * W))
    g = rng.standard_normal((B, T, D))
    return x, z, U, g


# ------------------------------------------------------------------ golden


def pin_golden_worked_examples(orc):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float64)
        g = np.array(c["dy"], dtype=np.float64)
        cu = c["cu_seqlens"]
        if c["kind"] == "headwise":
            w = np.array(c["w"], dtype=np.float64)
            y = orc.headwise_fwd(x, w, cu_seqlens=cu, residual=c["residual"])
            dx, dw = orc.headwise_bwd(x, w, g, cu_seqlens=cu, residual=c["residual"])
            _close(y, c["y"], what=c["name"] + " y")
            _close(dx, c["dx"], what=c["name"] + " dx")
            _close(dw, c["dw"], what=c["name"] + " dw")
        else:
            z = np.array(c["z"], dtype=np.float64)
            U = np.array(c["U"], dtype=np.float64)
            y = orc.lowrank_fwd(x, z, U, c["W"], cu_seqlens=cu, residual=c["residual"])
            dx, dz, dU = orc.lowrank_bwd(x, z, U, g, c["W"], cu_seqlens=cu, residual=c["residual"])
            _close(y, c["y"], what=c["name"] + " y")
            _close(dx, c["dx"], what=c["name"] + " dx")
            _close(dz, c["dz"], what=c["name"] + " dz")
            _close(dU, c["dU"], what=c["name"] + " dU")


# ------------------------------------------------------------- brute force


def pin_bruteforce_headwise(orc):
    rng = _rng(1)
    for (B, T, D, W, H, cu, res) in [(2, 9, 8, 4, 2, None, False), (1, 11, 6, 3, 3, [0, 4, 5, 11], True),
                                     (2, 5, 4, 4, 1, [0, 2, 5, 6, 10], False),
                                     (1, 7, 8, 8, 8, None, True)]:
        x, w, g = _hw_case(rng, B, T, D, W, H)
        seg = bf.seg_starts(B, T, cu)
        pc = bf.perchannel_filters_headwise(w, D)
        _close(orc.headwise_fwd(x, w, cu_seqlens=cu, residual=res), bf.conv_fwd(x, pc, seg, res),
               what="headwise y vs band matrix")
        dx, _ = orc.headwise_bwd(x, w, g, cu_seqlens=cu, residual=res)
        _close(dx, bf.conv_dx(g, pc, seg, res), what="headwise dx vs band matrix transpose")


def pin_bruteforce_lowrank(orc):
    rng = _rng(2)
    for (B, T, D, W, R, cu, res) in [(2, 7, 4, 4, 3, None, False), (1, 10, 5, 3, 2, [0, 3, 4, 10], True),
                                     (1, 6, 2, 1, 4, None, True)]:
        x, z, U, g = _lr_case(rng, B, T, D, W, R)
        seg = bf.seg_starts(B, T, cu)
        pc = bf.perchannel_filters_lowrank(z, U, W)
        _close(orc.lowrank_fwd(x, z, U, W, cu_seqlens=cu, residual=res), bf.conv_fwd(x, pc, seg, res),
               what="lowrank y vs band matrix")
        dx, dz, dU = orc.lowrank_bwd(x, z, U, g, W, cu_seqlens=cu, residual=res)
        _close(dx, bf.conv_dx(g, pc, seg, res), what="lowrank dx vs band matrix transpose")
        # dz, dU through the per-channel filter gradient of the brute force:
        # dL/dw_pc[n,d,k] = g[n,d] * (A_d's column shift of x)[n] (band entries only)
        N = B * T
        gf, xf = g.reshape(N, D), x.reshape(N, D)
        dwpc = np.zeros((N, D, W))
        for n in range(N):
            for k in range(W):
                if n - k >= seg[n]:
                    dwpc[n, :, k] = gf[n] * xf[n - k]
        _close(dz.reshape(N, R), np.einsum("ndk,rdk->nr", dwpc, U.reshape(R, D, W)), what="lowrank dz chain")
        _close(dU, np.einsum("nr,ndk->rdk", z.reshape(N, R), dwpc).reshape(R, D * W), what="lowrank dU chain")


# ------------------------------------------------------------ closed forms


def pin_impulse_response(orc):
    """x = e_(s,d): y_t[d] = w_t[j(d), t-s] for 0 <= t-s < W (same segment), else 0."""
    rng = _rng(3)
    B, T, D, W, H = 1, 10, 6, 4, 3
    w = rng.standard_normal((B, T, D // H, W))
    for s in (0, 3, 8):
        for d in (0, 4):
            x = np.zeros((B, T, D))
            x[0, s, d] = 1.0
            y = orc.headwise_fwd(x, w)
            want = np.zeros((B, T, D))
            for t in range(s, min(s + W, T)):
                want[0, t, d] = w[0, t, d // H, t - s]
            _close(y, want, what=f"impulse s={s} d={d}")


def pin_static_filter_is_numpy_convolve(orc):
    """Constant filters over time: the op is the static causal conv (numpy.convolve, truncated)."""
    rng = _rng(4)
    B, T, D, W, H = 2, 13, 4, 4, 2
    c = rng.standard_normal((D // H, W))
    w = np.broadcast_to(c, (B, T, D // H, W)).copy()
    x = rng.standard_normal((B, T, D))
    y = orc.headwise_fwd(x, w)
    for b in range(B):
        for d in range(D):
            _close(y[b, :, d], np.convolve(x[b, :, d], c[d // H])[:T], what="static conv")
    # low-rank with constant z: static filter z0 U
    R = 3
    z0 = rng.standard_normal(R)
    U = rng.standard_normal((R, D * W))
    z = np.broadcast_to(z0, (B, T, R)).copy()
    y = orc.lowrank_fwd(x, z, U, W)
    filt = (z0 @ U).reshape(D, W)
    for b in range(B):
        for d in range(D):
            _close(y[b, :, d], np.convolve(x[b, :, d], filt[d])[:T], what="static conv low-rank")
    # static dx is the correlation with the same filter (flip of convolve)
    g = rng.standard_normal((B, T, D))
    dx, _ = orc.headwise_bwd(x, w, g)
    for b in range(B):
        for d in range(D):
            full = np.convolve(g[b, ::-1, d], c[d // H])[:T][::-1]
            _close(dx[b, :, d], full, what="static dx")


def pin_width_one_is_scaling(orc):
    rng = _rng(5)
    B, T, D, H = 2, 6, 8, 4
    x = rng.standard_normal((B, T, D))
    w = rng.standard_normal((B, T, D // H, 1))
    g = rng.standard_normal((B, T, D))
    scale = np.repeat(w[..., 0], H, axis=2)
    for res in (False, True):
        y = orc.headwise_fwd(x, w, residual=res)
        _close(y, (res + scale) * x, what="W=1 y")
        dx, dw = orc.headwise_bwd(x, w, g, residual=res)
        _close(dx, (res + scale) * g, what="W=1 dx")
        _close(dw[..., 0], (g * x).reshape(B, T, D // H, H).sum(-1), what="W=1 dw")


def pin_rank_one_closed_form(orc):
    """R = 1: y_t[d] = z_t * (x[:, d] convolved with U[0, d, :])_t."""
    rng = _rng(6)
    B, T, D, W = 1, 12, 3, 4
    x = rng.standard_normal((B, T, D))
    z = rng.standard_normal((B, T, 1))
    U = rng.standard_normal((1, D * W))
    y = orc.lowrank_fwd(x, z, U, W)
    for d in range(D):
        conv = np.convolve(x[0, :, d], U[0].reshape(D, W)[d])[:T]
        _close(y[0, :, d], z[0, :, 0] * conv, what="rank-1")


def pin_headwise_equals_perchannel(orc):
    rng = _rng(7)
    B, T, D, W, H = 2, 8, 8, 3, 4
    x, w, g = _hw_case(rng, B, T, D, W, H)
    wpc = np.repeat(w, H, axis=2)
    _close(orc.headwise_fwd(x, w, residual=True), orc.headwise_fwd(x, wpc, residual=True),
           what="head-wise == per-channel y")
    dx_h, dw_h = orc.headwise_bwd(x, w, g)
    dx_p, dw_p = orc.headwise_bwd(x, wpc, g)
    _close(dx_h, dx_p, what="head-wise == per-channel dx")
    _close(dw_h, dw_p.reshape(B, T, D // H, H, W).sum(3), what="dw == group sum of per-channel dw")


# ------------------------------------------------ adjoint / finite differences


def pin_adjoint_identity(orc):
    rng = _rng(8)
    B, T, D, W, H = 2, 9, 4, 4, 2
    cu = [0, 3, 9, 12, 18]
    x, w, g = _hw_case(rng, B, T, D, W, H)
    y = orc.headwise_fwd(x, w, cu_seqlens=cu)
    dx, _ = orc.headwise_bwd(x, w, g, cu_seqlens=cu)
    lhs, rhs = float(np.sum(g * y)), float(np.sum(dx * x))
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), f"adjoint {lhs} vs {rhs}"
    R = 3
    xl, z, U, gl = _lr_case(rng, B, T, D, W, R)
    y = orc.lowrank_fwd(xl, z, U, W, cu_seqlens=cu)
    dx, dz, dU = orc.lowrank_bwd(xl, z, U, gl, W, cu_seqlens=cu)
    L = float(np.sum(gl * y))
    for name, v in (("x", np.sum(dx * xl)), ("z", np.sum(dz * z)), ("U", np.sum(dU * U))):
        # y is linear (degree-1 homogeneous) in each of x, z, U separately
        assert abs(L - float(v)) <= 1e-11 * max(1.0, abs(L)), f"Euler identity in {name}: {L} vs {v}"


def _fd_grad(f, a, h=1e-3):
    grad = np.zeros_like(a)
    flat, gflat = a.reshape(-1), grad.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        fp = f()
        flat[i] = old - h
        fm = f()
        flat[i] = old
        gflat[i] = (fp - fm) / (2 * h)
    return grad


def pin_finite_differences_headwise(orc):
    rng = _rng(9)
    B, T, D, W, H = 2, 6, 4, 3, 2
    cu = [0, 4, 6, 12]
    x, w, g = _hw_case(rng, B, T, D, W, H)
    for res in (False, True):
        L = lambda: float(np.sum(g * orc.headwise_fwd(x, w, cu_seqlens=cu, residual=res)))
        dx, dw = orc.headwise_bwd(x, w, g, cu_seqlens=cu, residual=res)
        _close(dx, _fd_grad(L, x), tol=1e-8, what="FD dx")
        _close(dw, _fd_grad(L, w), tol=1e-8, what="FD dw")


def pin_finite_differences_lowrank(orc):
    rng = _rng(10)
    B, T, D, W, R = 2, 5, 3, 3, 2
    cu = [0, 2, 5, 7, 10]
    x, z, U, g = _lr_case(rng, B, T, D, W, R)
    for res in (False, True):
        L = lambda: float(np.sum(g * orc.lowrank_fwd(x, z, U, W, cu_seqlens=cu, residual=res)))
        dx, dz, dU = orc.lowrank_bwd(x, z, U, g, W, cu_seqlens=cu, residual=res)
        _close(dx, _fd_grad(L, x), tol=1e-8, what="FD dx low-rank")
        _close(dz, _fd_grad(L, z), tol=1e-8, what="FD dz")
        _close(dU, _fd_grad(L, U), tol=1e-8, what="FD dU")


# ------------------------------------------------------- structural identities


def pin_segments_are_independent(orc):
    """Packed result == every segment run alone as its own sequence (dU sums over segments)."""
    rng = _rng(11)
    B, T, D, W, H, R = 2, 10, 4, 4, 2, 3
    cu = [0, 1, 4, 10, 13, 20]
    x, w, g = _hw_case(rng, B, T, D, W, H)
    y = orc.headwise_fwd(x, w, cu_seqlens=cu, residual=True).reshape(B * T, D)
    dx, dw = orc.headwise_bwd(x, w, g, cu_seqlens=cu, residual=True)
    dx, dw = dx.reshape(B * T, D), dw.reshape(B * T, D // H, W)
    xf, wf, gf = x.reshape(B * T, D), w.reshape(B * T, D // H, W), g.reshape(B * T, D)
    xl, z, U, gl = _lr_case(rng, B, T, D, W, R)
    yl = orc.lowrank_fwd(xl, z, U, W, cu_seqlens=cu).reshape(B * T, D)
    dxl, dzl, dUl = orc.lowrank_bwd(xl, z, U, gl, W, cu_seqlens=cu)
    dxl, dzl = dxl.reshape(B * T, D), dzl.reshape(B * T, R)
    xlf, zf, glf = xl.reshape(B * T, D), z.reshape(B * T, R), gl.reshape(B * T, D)
    dU_sum = np.zeros_like(dUl)
    for a, b in zip(cu[:-1], cu[1:]):
        L = b - a
        ys = orc.headwise_fwd(xf[None, a:b], wf[None, a:b], residual=True)[0]
        dxs, dws = orc.headwise_bwd(xf[None, a:b], wf[None, a:b], gf[None, a:b], residual=True)
        _close(y[a:b], ys, what=f"segment [{a},{b}) y")
        _close(dx[a:b], dxs[0], what=f"segment [{a},{b}) dx")
        _close(dw[a:b], dws[0], what=f"segment [{a},{b}) dw")
        ysl = orc.lowrank_fwd(xlf[None, a:b], zf[None, a:b], U, W)[0]
        dxs, dzs, dUs = orc.lowrank_bwd(xlf[None, a:b], zf[None, a:b], U, glf[None, a:b], W)
        _close(yl[a:b], ysl, what=f"segment [{a},{b}) low-rank y")
        _close(dxl[a:b], dxs[0], what=f"segment [{a},{b}) low-rank dx")
        _close(dzl[a:b], dzs[0], what=f"segment [{a},{b}) dz")
        dU_sum += dUs
        assert L >= 1
    _close(dUl, dU_sum, what="dU = sum over segments")


def pin_locality_and_causality(orc):
    """Changing x[s] changes y only at tokens s .. min(s+W-1, end of s's segment)."""
    rng = _rng(12)
    B, T, D, W, H = 1, 16, 2, 4, 1
    cu = [0, 6, 16]
    x, w, _ = _hw_case(rng, B, T, D, W, H)
    y0 = orc.headwise_fwd(x, w, cu_seqlens=cu)
    for s in (0, 4, 5, 6, 14):
        x1 = x.copy()
        x1[0, s, 1] += 1.0
        diff = np.abs(orc.headwise_fwd(x1, w, cu_seqlens=cu) - y0)[0]
        end = 6 if s < 6 else 16
        changed = set(np.nonzero(diff.max(axis=1) > 0)[0].tolist())
        allowed = set(range(s, min(s + W, end)))
        assert changed <= allowed, f"x[{s}] changed tokens {sorted(changed)} outside {sorted(allowed)}"
        assert s in changed, f"x[{s}] did not change y[{s}]"
        assert np.all(diff[:, 0] == 0), "another channel changed"


def pin_row_ranges_match_full(orc):
    """Computing a token range / channel range gives the same values as the full call."""
    rng = _rng(13)
    B, T, D, W, R = 2, 7, 4, 4, 2
    x, z, U, g = _lr_case(rng, B, T, D, W, R)
    dx, dz, dU = orc.lowrank_bwd(x, z, U, g, W, residual=True)
    dxr, dzr, dUr = orc.lowrank_bwd(x, z, U, g, W, residual=True, rows=(3, 11), channels=(1, 3))
    _close(dxr, dx.reshape(B * T, D)[3:11], what="row range dx")
    _close(dzr, dz.reshape(B * T, R)[3:11], what="row range dz")
    _close(dUr, dU.reshape(R, D, W)[:, 1:3].reshape(R, 2 * W), what="channel range dU")


# ------------------------------------------------------------ static filter
# The fixed-filter layer the dynamic convolution generalises (authors' thread
# on digg.com): one filter c[d, :] per channel, the same at every position.


def pin_static_layer_is_numpy_convolve(orc):
    """Per sequence and channel: y = rho*x + numpy.convolve(x, c[d])[:L], dx the same
    with the sequence reversed, dc[d, k] the lag-k entry of numpy.correlate(g, x)."""
    rng = _rng(14)
    B, T, D, W = 2, 11, 5, 4
    cu = [0, 1, 4, 11, 13, 22]
    x = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D))
    c = rng.standard_normal((D, W))
    for res in (False, True):
        y = orc.static_fwd(x, c, cu_seqlens=cu, residual=res).reshape(B * T, D)
        dx, dc = orc.static_bwd(x, c, g, cu_seqlens=cu, residual=res)
        dx = dx.reshape(B * T, D)
        xf, gf = x.reshape(B * T, D), g.reshape(B * T, D)
        want_dc = np.zeros((D, W))
        for a, b in zip(cu[:-1], cu[1:]):
            L = b - a
            for d in range(D):
                _close(y[a:b, d], res * xf[a:b, d] + np.convolve(xf[a:b, d], c[d])[:L], what="static y")
                _close(dx[a:b, d], res * gf[a:b, d] + np.convolve(gf[a:b, d][::-1], c[d])[:L][::-1],
                       what="static dx")
                corr = np.correlate(gf[a:b, d], xf[a:b, d], mode="full")  # index L-1+k <-> lag k
                for k in range(min(W, L)):
                    want_dc[d, k] += corr[L - 1 + k]
        _close(dc, want_dc, what="static dc")


def pin_static_equals_constant_filter(orc):
    """The static layer is the per-channel dynamic one with the same filter at every token."""
    rng = _rng(15)
    B, T, D, W = 2, 9, 6, 3
    cu = [0, 5, 7, 18]
    x = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D))
    c = rng.standard_normal((D, W))
    w = np.broadcast_to(c, (B, T, D, W)).copy()
    _close(orc.static_fwd(x, c, cu_seqlens=cu, residual=True),
           orc.headwise_fwd(x, w, cu_seqlens=cu, residual=True), what="static == constant dynamic y")
    dx_s, dc = orc.static_bwd(x, c, g, cu_seqlens=cu, residual=True)
    dx_h, dw = orc.headwise_bwd(x, w, g, cu_seqlens=cu, residual=True)
    _close(dx_s, dx_h, what="static == constant dynamic dx")
    _close(dc, dw.reshape(B * T, D, W).sum(0), what="dc == sum over tokens of the per-token dw")


def pin_static_width_one_is_scaling(orc):
    rng = _rng(16)
    B, T, D = 2, 5, 3
    x = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D))
    c = rng.standard_normal((D, 1))
    for res in (False, True):
        _close(orc.static_fwd(x, c, residual=res), (res + c[:, 0]) * x, what="static W=1 y")
        dx, dc = orc.static_bwd(x, c, g, residual=res)
        _close(dx, (res + c[:, 0]) * g, what="static W=1 dx")
        _close(dc[:, 0], (g * x).sum(axis=(0, 1)), what="static W=1 dc")


def pin_finite_differences_static(orc):
    rng = _rng(17)
    B, T, D, W = 2, 5, 3, 4
    cu = [0, 3, 4, 10]
    x = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D))
    c = rng.standard_normal((D, W))
    for res in (False, True):
        L = lambda: float(np.sum(g * orc.static_fwd(x, c, cu_seqlens=cu, residual=res)))
        dx, dc = orc.static_bwd(x, c, g, cu_seqlens=cu, residual=res)
        _close(dx, _fd_grad(L, x), tol=1e-8, what="FD static dx")
        _close(dc, _fd_grad(L, c), tol=1e-8, what="FD static dc")


# ---------------------------------------------------------------- decoding
# One token per sequence with a rolling state of the last W-1 inputs: the
# step is the forward evaluated at the sequence's newest token.


def pin_decode_reproduces_forward(orc):
    """Decoding a sequence token by token from a zero state gives the forward at
    every position (head-wise and low-rank), and leaves the prefill state."""
    rng = _rng(18)
    B, T, D, W, H, R = 3, 9, 8, 4, 2, 3
    x, w, _ = _hw_case(rng, B, T, D, W, H)
    xl, z, U, _ = _lr_case(rng, B, T, D, W, R)
    for res in (False, True):
        y = orc.headwise_fwd(x, w, residual=res)
        yl = orc.lowrank_fwd(xl, z, U, W, residual=res)
        st = np.zeros((B, W - 1, D))
        stl = np.zeros((B, W - 1, D))
        for t in range(T):
            yt, st = orc.headwise_decode(x[:, t], w[:, t], st, residual=res)
            _close(yt, y[:, t], what=f"head-wise decode t={t}")
            ylt, stl = orc.lowrank_decode(xl[:, t], z[:, t], U, stl, W, residual=res)
            _close(ylt, yl[:, t], what=f"low-rank decode t={t}")
        _close(st, orc.state_from_prefill(x, W), what="state after decoding == prefill state")
        _close(stl, orc.state_from_prefill(xl, W), what="low-rank state == prefill state")


def pin_prefill_handoff(orc):
    """Packed prefill (sequences of 1..6 tokens, some shorter than W-1), state
    from the prefill, then decode steps: the same outputs as the forward over
    the whole sequences."""
    rng = _rng(19)
    D, W, H, steps = 4, 5, 1, 3
    lens = [1, 6, 2, 4]
    S = len(lens)
    full = [rng.standard_normal((L + steps, D)) for L in lens]
    wf = [rng.standard_normal((L + steps, D // H, W)) for L in lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    xp = np.concatenate([f[:L] for f, L in zip(full, lens)])[None]
    st = orc.state_from_prefill(xp, W, cu_seqlens=cu)
    assert st.shape == (S, W - 1, D)
    for j in range(steps):
        xt = np.stack([f[L + j] for f, L in zip(full, lens)])
        wt = np.stack([g[L + j] for g, L in zip(wf, lens)])
        yt, st = orc.headwise_decode(xt, wt, st, residual=True)
        for s_, (f, g, L) in enumerate(zip(full, wf, lens)):
            want = orc.headwise_fwd(f[None, :L + j + 1], g[None, :L + j + 1], residual=True)[0, -1]
            _close(yt[s_], want, what=f"hand-off sequence {s_} step {j}")


# --------------------------------------------------------- rotary positions
# The rotation that the placement puts right after the layer on queries and
# keys is RoFormer's ("RoFormer: Enhanced Transformer with Rotary Position
# Embedding", Su et al., Section 3.4.2): pair i = channels (2i, 2i+1) of a head
# of hd channels turns by m * theta_i at position m, theta_i = base^(-2i/hd).

# cos and sin of 1, 2 and 10 radians (standard tables, 17 significant digits)
_COS1, _SIN1 = 0.54030230586813972, 0.84147098480789651
_COS2, _SIN2 = -0.41614683654714239, 0.90929742682568170
_COS10, _SIN10 = -0.83907152907645245, -0.54402111088936981


def pin_rope_worked_values(orc):
    """Unit vectors through the rotation at positions whose angles are whole
    radians, and the cos / sin table at the same points."""
    # head_dim 2: theta_0 = 1 for any base, so position m turns by m radians
    for e, want in ((0, [[1, 0], [_COS1, _SIN1], [_COS2, _SIN2]]),
                    (1, [[0, 1], [-_SIN1, _COS1], [-_SIN2, _COS2]])):
        v = np.zeros((1, 3, 2))
        v[0, :, e] = 1.0
        _close(orc.rope(v, rot=2, head_dim=2, base=5.0)[0], want, what=f"head_dim 2, unit vector {e}")
    # head_dim 4, base 100: theta_0 = 1 and theta_1 = 100^(-1/2) = 0.1, so at
    # position 10 pair 0 turns by 10 rad and pair 1 by 1 rad.  Two rotated
    # heads (channels 0..7), then one value channel that passes unchanged.
    v = np.zeros((1, 11, 9))
    v[0, :, 0] = 1.0  # head 0, pair 0
    v[0, :, 6] = 1.0  # head 1, pair 1
    v[0, :, 8] = 3.0
    out = orc.rope(v, rot=8, head_dim=4, base=100.0)[0, 10]
    _close(out, [_COS10, _SIN10, 0, 0, 0, 0, _COS1, _SIN1, 3.0], what="head_dim 4, base 100, position 10")
    _close(orc.rope_table(3, 2, base=7.0)[:, 0], [[1, 0], [_COS1, _SIN1], [_COS2, _SIN2]], what="table, head_dim 2")
    _close(orc.rope_table(11, 4, base=100.0)[10], [[_COS10, _SIN10], [_COS1, _SIN1]], what="table, head_dim 4")


def pin_rope_relative_positions(orc):
    """RoFormer's defining property: the inner product of a rotated query at
    position m and a rotated key at position n depends on m - n only; and the
    rotation keeps the norm of every head."""
    rng = _rng(20)
    hd, heads, T = 8, 2, 12
    q, k = rng.standard_normal(heads * hd), rng.standard_normal(heads * hd)
    v = np.tile(np.concatenate([q, k]), (1, T, 1))  # every token holds the same q and k
    r = orc.rope(v, rot=2 * heads * hd, head_dim=hd, base=50.0)[0]
    rq, rk = r[:, :heads * hd], r[:, heads * hd:]
    for m, n in ((2, 0), (5, 7), (4, 4), (0, 9)):
        for shift in (1, 2):
            assert abs(rq[m] @ rk[n] - rq[m + shift] @ rk[n + shift]) <= 1e-12 * (abs(q) @ abs(k)), \
                f"<q_m, k_n> changed under a common shift of m={m}, n={n}"
    _close(rq[3] @ rk[3], q @ k, what="equal positions give the unrotated product")
    _close(np.linalg.norm(r.reshape(T, -1, hd), axis=-1), np.linalg.norm(v[0].reshape(T, -1, hd), axis=-1),
           what="head norms")


def pin_rope_segments_inverse_passthrough(orc):
    """Positions restart at every packed sequence (packed rows equal each
    sequence rotated alone); channels from rot on pass unchanged; the inverse
    undoes the rotation; compact row ranges match the full result."""
    rng = _rng(21)
    B, T, D, hd, rot = 2, 7, 20, 4, 12
    cu = [0, 3, 7, 14]
    x = rng.standard_normal((B, T, D))
    r = orc.rope(x, rot=rot, head_dim=hd, base=9.0, cu_seqlens=cu)
    flat, xf = r.reshape(B * T, D), x.reshape(B * T, D)
    for a, b in zip(cu[:-1], cu[1:]):
        _close(flat[a:b], orc.rope(xf[None, a:b], rot=rot, head_dim=hd, base=9.0)[0], what=f"segment [{a},{b})")
    _close(r[..., rot:], x[..., rot:], what="channels past rot")
    _close(orc.rope(r, rot=rot, head_dim=hd, base=9.0, cu_seqlens=cu, inverse=True), x, what="inverse")
    part = orc.rope(xf[5:11], rot=rot, head_dim=hd, base=9.0, cu_seqlens=cu, rows=(5, 11), shape=(B, T))
    _close(part, flat[5:11], what="row range")


def pin_rope_layer_composition(orc):
    """rot = 0 leaves the head-wise layer unchanged; the fused layer's
    gradients equal exact central finite differences of L = <g, y>."""
    rng = _rng(22)
    B, T, D, W, H, hd = 2, 5, 8, 3, 2, 4
    cu = [0, 3, 5, 10]
    x, w, g = _hw_case(rng, B, T, D, W, H)
    _close(orc.headwise_rope_fwd(x, w, rot=0, head_dim=hd, residual=True, cu_seqlens=cu),
           orc.headwise_fwd(x, w, residual=True, cu_seqlens=cu), what="rot = 0")
    for res in (False, True):
        f = lambda: float(np.sum(g * orc.headwise_rope_fwd(x, w, rot=4, head_dim=hd, base=3.0, cu_seqlens=cu,
                                                            residual=res)))
        dx, dw = orc.headwise_rope_bwd(x, w, g, rot=4, head_dim=hd, base=3.0, cu_seqlens=cu, residual=res)
        _close(dx, _fd_grad(f, x), tol=1e-8, what="FD dx (RoPE)")
        _close(dw, _fd_grad(f, w), tol=1e-8, what="FD dw (RoPE)")


def pin_rope_lowrank_layer_composition(orc):
    """The low-rank layer followed by the rotation: rot = 0 leaves the layer
    unchanged, the rotated output is the layer's output turned pair by pair
    (checked against the rotation alone on the layer's output rows), and the
    fused gradients dx, dz, dU equal exact central finite differences of
    L = <g, y> (L is linear in x, in z and in U)."""
    rng = _rng(24)
    B, T, D, W, R, hd = 2, 5, 8, 3, 2, 4
    cu = [0, 2, 5, 10]
    x, z, U, g = _lr_case(rng, B, T, D, W, R)
    _close(orc.lowrank_rope_fwd(x, z, U, W, rot=0, head_dim=hd, residual=True, cu_seqlens=cu),
           orc.lowrank_fwd(x, z, U, W, residual=True, cu_seqlens=cu), what="rot = 0")
    # value channels [rot, D) pass unchanged; query / key channels keep their norm per pair
    y0 = orc.lowrank_fwd(x, z, U, W, cu_seqlens=cu)
    y1 = orc.lowrank_rope_fwd(x, z, U, W, rot=4, head_dim=hd, base=3.0, cu_seqlens=cu)
    _close(y1[..., 4:], y0[..., 4:], what="channels past rot")
    _close(np.hypot(y1[..., 0:4:2], y1[..., 1:4:2]), np.hypot(y0[..., 0:4:2], y0[..., 1:4:2]), what="pair norms")
    for res in (False, True):
        f = lambda: float(np.sum(g * orc.lowrank_rope_fwd(x, z, U, W, rot=4, head_dim=hd, base=3.0, cu_seqlens=cu,
                                                           residual=res)))
        dx, dz, dU = orc.lowrank_rope_bwd(x, z, U, g, W, rot=4, head_dim=hd, base=3.0, cu_seqlens=cu,
                                          residual=res)
        _close(dx, _fd_grad(f, x), tol=1e-8, what="FD dx (low-rank, RoPE)")
        _close(dz, _fd_grad(f, z), tol=1e-8, what="FD dz (low-rank, RoPE)")
        _close(dU, _fd_grad(f, U), tol=1e-8, what="FD dU (low-rank, RoPE)")


def pin_rope_decode_reproduces_forward(orc):
    """Decoding with the rotation at each token's position, after a packed
    prefill of sequences of 1..6 tokens, gives the fused forward over the
    whole sequences; positions restart per sequence."""
    rng = _rng(23)
    D, W, H, hd, rot, steps = 12, 3, 2, 4, 8, 3
    lens = [1, 6, 2, 4]
    full = [rng.standard_normal((L + steps, D)) for L in lens]
    wf = [rng.standard_normal((L + steps, D // H, W)) for L in lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    xp = np.concatenate([f[:L] for f, L in zip(full, lens)])[None]
    st = orc.state_from_prefill(xp, W, cu_seqlens=cu)
    for j in range(steps):
        xt = np.stack([f[L + j] for f, L in zip(full, lens)])
        wt = np.stack([g[L + j] for g, L in zip(wf, lens)])
        pos = np.array([L + j for L in lens])
        yt, st = orc.headwise_rope_decode(xt, wt, st, pos, rot=rot, head_dim=hd, base=7.0, residual=True)
        for s_, (f, g, L) in enumerate(zip(full, wf, lens)):
            want = orc.headwise_rope_fwd(f[None, :L + j + 1], g[None, :L + j + 1], rot=rot, head_dim=hd,
                                         base=7.0, residual=True)[0, -1]
            _close(yt[s_], want, what=f"rotated decode, sequence {s_} step {j}")


# ------------------------------------------------------- filter generator


def _gen_case(rng, B, T, D, W, H, K):
    h = rng.standard_normal((B, T, K))
    V = rng.standard_normal(((D // H) * W, K))
    x = rng.standard_normal((B, T, D))
    g = rng.standard_normal((B, T, D))
    return h, V, x, g


def pin_generator_bruteforce(orc):
    """The generated filters and the layer on them, by direct loops over
    every index (the map w[n, g*W + k] = sum_j h[n, j] V[g*W + k, j], then
    the convolution with the per-sequence causal mask); the map alone also
    against numpy's matrix product."""
    rng = _rng(30)
    B, T, D, W, H, K = 2, 5, 6, 3, 2, 4
    cu = [0, 2, 5, 7, 10]
    h, V, x, _ = _gen_case(rng, B, T, D, W, H, K)
    hf, xf = h.reshape(-1, K), x.reshape(-1, D)
    _close(orc.generate(h, V), hf @ V.T, what="generator == h V^T")
    seg = np.zeros(B * T, dtype=int)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        seg[s0:s1] = s0
    for res in (False, True):
        want = np.zeros((B * T, D))
        for n in range(B * T):
            for d in range(D):
                acc = xf[n, d] if res else 0.0
                for k in range(W):
                    if n - k >= seg[n]:
                        wk = sum(hf[n, j] * V[(d // H) * W + k, j] for j in range(K))
                        acc += wk * xf[n - k, d]
                want[n, d] = acc
        got = orc.headwise_gen_fwd(h, V, x, W=W, cu_seqlens=cu, residual=res)
        _close(got.reshape(-1, D), want, what=f"generated layer, residual={res}")


def pin_generator_finite_differences(orc):
    """dx, dh, dV of L = <g, y> equal exact central differences (L is linear
    in each of h, V and x separately)."""
    rng = _rng(31)
    B, T, D, W, H, K = 2, 4, 4, 3, 2, 3
    cu = [0, 3, 4, 8]
    h, V, x, g = _gen_case(rng, B, T, D, W, H, K)
    for res in (False, True):
        f = lambda: float(np.sum(g * orc.headwise_gen_fwd(h, V, x, W=W, cu_seqlens=cu, residual=res)))
        dx, dh, dV = orc.headwise_gen_bwd(h, V, x, g, W=W, cu_seqlens=cu, residual=res)
        _close(dx, _fd_grad(f, x), tol=1e-8, what="FD dx (generated)")
        _close(dh, _fd_grad(f, h), tol=1e-8, what="FD dh")
        _close(dV, _fd_grad(f, V), tol=1e-8, what="FD dV")


def pin_generator_constant_state_is_static(orc):
    """A hidden state that is the same unit vector e_0 at every token makes
    the filter the same at every token, w = V[:, 0]: the layer is then the
    static short convolution with c[d, k] = V[(d/H)*W + k, 0], dV[:, 0] is
    the static filter gradient summed over each group's channels, and dV is
    zero in every other column."""
    rng = _rng(32)
    B, T, D, W, H, K = 2, 7, 6, 4, 3, 3
    cu = [0, 5, 9, 14]
    _, V, x, g = _gen_case(rng, B, T, D, W, H, K)
    h = np.zeros((B, T, K))
    h[..., 0] = 1.0
    c = np.repeat(V[:, 0].reshape(D // H, W), H, axis=0)
    _close(orc.headwise_gen_fwd(h, V, x, W=W, cu_seqlens=cu, residual=True),
           orc.static_fwd(x, c, cu_seqlens=cu, residual=True), what="constant state == static layer")
    dx, dh, dV = orc.headwise_gen_bwd(h, V, x, g, W=W, cu_seqlens=cu, residual=True)
    sdx, sdc = orc.static_bwd(x, c, g, cu_seqlens=cu, residual=True)
    _close(dx, sdx, what="constant state dx == static dx")
    _close(dV[:, 0], sdc.reshape(D // H, H, W).sum(1).reshape(-1), what="dV column 0 == grouped static dc")
    _close(dV[:, 1:], np.zeros_like(dV[:, 1:]), what="dV of unused state columns")


def pin_generator_rows_and_groups_match_full(orc):
    rng = _rng(33)
    B, T, D, W, H, K = 2, 9, 8, 3, 2, 5
    cu = [0, 4, 9, 10, 18]
    h, V, x, g = _gen_case(rng, B, T, D, W, H, K)
    N = B * T
    y = orc.headwise_gen_fwd(h, V, x, W=W, cu_seqlens=cu, residual=True).reshape(N, D)
    dx, dh, dV = orc.headwise_gen_bwd(h, V, x, g, W=W, cu_seqlens=cu, residual=True)
    dx, dh = dx.reshape(N, D), dh.reshape(N, K)
    for lo, hi in [(0, 3), (5, 12), (N - 2, N), (7, 7)]:
        _close(orc.headwise_gen_fwd(h, V, x, W=W, cu_seqlens=cu, residual=True, rows=(lo, hi)), y[lo:hi],
               what=f"y rows {lo}:{hi}")
        rdx, rdh, rdV = orc.headwise_gen_bwd(h, V, x, g, W=W, cu_seqlens=cu, residual=True, rows=(lo, hi),
                                             groups=(1, 3))
        _close(rdx, dx[lo:hi], what=f"dx rows {lo}:{hi}")
        _close(rdh, dh[lo:hi], what=f"dh rows {lo}:{hi}")
        _close(rdV, dV[W:3 * W], what="dV groups 1:3")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
