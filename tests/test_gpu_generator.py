"""GPU parity of the head-wise layer whose filters are generated on chip from
the hidden state (w = h V^T, the learned linear map of the pages'
parametrization), through the C ABI against the fp64 oracle.

y, dx, dh and dV are compared element by element at small shapes (every tap
count, several group sizes including ones that are not a multiple of 8, group
tiles cut at the end, packed sequences, h = x), and at the MLP ~2B head-wise
shape (B=4 T=4096 D=8192 W=4 H=16, hidden width 2048) and the QKV ~150M shape
(B=8 T=2048 D=2304 W=4 H=64, hidden width 768) on token windows and group
blocks, with the bf16 normwise tolerance 2e-2.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, Guarded, assert_close, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu


def _run(inp, W, H, res, *, h_is_x=False):
    x, dy, V = (inp[k].cuda() for k in ("x", "dy", "V"))
    h = x if h_is_x else inp["h"].cuda()
    B, T, D = x.shape
    K = h.shape[2]
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    y, dx, dh = Guarded(x.shape, x.dtype), Guarded(x.shape, x.dtype), Guarded(h.shape, h.dtype)
    dV = Guarded(V.shape, torch.float32)
    nws = binding.dsc_headwise_gen_bwd_workspace_size(x.dtype, B, T, D, W, H, K)
    ws = torch.full((nws // 2,), float("nan"), dtype=torch.bfloat16, device="cuda")
    binding.dsc_headwise_gen_fwd(h, V, x, y.t, W=W, cu_seqlens=cu, residual=res)
    binding.dsc_headwise_gen_bwd(h, V, x, dy, dx.t, dh.t, dV.t, ws, W=W, cu_seqlens=cu, residual=res)
    torch.cuda.synchronize()
    for name, g in (("y", y), ("dx", dx), ("dh", dh), ("dV", dV)):
        g.check_guards(name)
    return y, dx, dh, dV


# (B, T, D, W, H, K, residual, segment-length range or None)
GEN_CASES = [
    (2, 37, 64, 4, 16, 32, True, None),
    (1, 150, 128, 3, 8, 64, False, (1, 40)),
    (1, 300, 512, 4, 16, 256, True, (1, 100)),    # three token tiles, one whole group tile
    (2, 200, 1024, 4, 16, 128, False, None),      # two group tiles
    (1, 130, 96, 2, 3, 40, True, (1, 20)),        # groups of 3 channels: chunks straddle groups
    (1, 100, 2304, 4, 64, 768, True, None),       # QKV ~150M layout: 36 groups, last group tile cut
    (1, 90, 160, 5, 4, 24, True, (1, 30)),        # W = 5: tiles of 16 groups
    (1, 64, 64, 8, 8, 16, False, None),           # W = 8
    (1, 129, 256, 1, 16, 64, True, None),         # W = 1: no halo
    (1, 1, 64, 4, 16, 8, False, None),            # one token
    (3, 70, 192, 6, 12, 48, True, (1, 25)),       # W = 6, groups of 12
    (1, 260, 320, 7, 40, 72, False, (1, 90)),     # W = 7, groups of 40
]


def _ids(cases):
    return [f"gen-B{c[0]}T{c[1]}D{c[2]}W{c[3]}H{c[4]}K{c[5]}-res{int(c[6])}-{'varlen' if c[7] else 'rows'}"
            for c in cases]


def _check(inp, W, H, res, h_is_x=False):
    y, dx, dh, dV = _run(inp, W, H, res, h_is_x=h_is_x)
    cu = inp["cu_seqlens"]
    x64, g64, V64 = to_f64(inp["x"]), to_f64(inp["dy"]), to_f64(inp["V"])
    h64 = x64 if h_is_x else to_f64(inp["h"])
    kw = dict(W=W, cu_seqlens=cu, residual=res)
    tol = TOL["bf16"]
    assert_close("y", y.host(), oracle.headwise_gen_fwd(h64, V64, x64, **kw), tol)
    rdx, rdh, rdV = oracle.headwise_gen_bwd(h64, V64, x64, g64, **kw)
    assert_close("dx", dx.host(), rdx, tol)
    assert_close("dh", dh.host(), rdh, tol)
    assert_close("dV", dV.host(), rdV, tol)
    return y, dx, dh, dV


@pytest.mark.parametrize("case", GEN_CASES, ids=_ids(GEN_CASES))
def test_generated_headwise_small(case):
    B, T, D, W, H, K, res, seg = case
    wl, _ = inputs.small("headwise", B, T, D, W, H=H, dtype="bf16", residual=res, varlen=seg is not None,
                         seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    inp = inputs.generator_inputs(wl, K)
    say(f"[generator] {wl.name} K={K} residual={res} segments={inp['cu_seqlens']}")
    y, dx, dh, dV = _check(inp, W, H, res)
    # no atomics anywhere: a second run gives the same bits
    y2, dx2, dh2, dV2 = _run(inp, W, H, res)
    for a, b in ((y, y2), (dx, dx2), (dh, dh2), (dV, dV2)):
        assert torch.equal(a.t, b.t)


def test_generated_headwise_from_its_own_input():
    """h = x: the filters come from the layer's own input (the caller adds dh to dx)."""
    wl, _ = inputs.small("headwise", 2, 90, 256, 4, H=16, dtype="bf16", residual=True, varlen=True,
                         seglen_range=(1, 40), seed=41)
    inp = inputs.generator_inputs(wl, 256)
    say(f"[generator] {wl.name} h = x")
    _check(inp, 4, 16, True, h_is_x=True)


def test_generated_headwise_constant_state_is_the_layer():
    """A hidden state e_0 at every token gives w = V[:, 0] at every token: the
    output equals the head-wise layer run on those filters directly."""
    B, T, D, W, H, K = 2, 150, 256, 4, 16, 16
    wl, _ = inputs.small("headwise", B, T, D, W, H=H, dtype="bf16", residual=True, seed=42)
    inp = inputs.generator_inputs(wl, K)
    h = torch.zeros(B, T, K, dtype=torch.bfloat16)
    h[..., 0] = 1.0
    inp["h"] = h
    y, dx, _, _ = _run(inp, W, H, True)
    G = D // H
    w = inp["V"][:, 0].reshape(1, 1, G, W).expand(B, T, G, W).contiguous().cuda()
    y2, dx2, dw2 = torch.empty_like(inp["x"]).cuda(), torch.empty_like(inp["x"]).cuda(), torch.empty_like(w)
    binding.dsc_headwise_fwd(inp["x"].cuda(), w, y2, residual=True)
    binding.dsc_headwise_bwd(inp["x"].cuda(), w, inp["dy"].cuda(), dx2, dw2, residual=True)
    torch.cuda.synchronize()
    assert_close("y", y.host(), to_f64(y2), 2e-3)
    assert_close("dx", dx.host(), to_f64(dx2), 2e-3)


@pytest.mark.parametrize("N,K,C", [(300, 64, 48), (4096, 2048, 2048), (1, 8, 8), (1000, 40, 200)])
def test_generate_filters(N, K, C):
    """The generator alone (w written out) against the oracle's map; the
    fused forward on those filters equals the head-wise layer run on them."""
    g = torch.Generator().manual_seed(N + K + C)
    h = torch.randn(N, K, generator=g).to(torch.bfloat16)
    V = (torch.randn(C, K, generator=g) / np.sqrt(K)).to(torch.bfloat16)
    w = Guarded((N, C), torch.bfloat16)
    binding.dsc_generate_filters(h.cuda(), V.cuda(), w.t)
    torch.cuda.synchronize()
    w.check_guards("w")
    say(f"[generator] filters N={N} K={K} C={C}")
    assert_close("w", w.host(), oracle.generate(to_f64(h), to_f64(V)), TOL["bf16"])


def test_generated_headwise_empty_batch():
    x = torch.empty(0, 16, 64, dtype=torch.bfloat16, device="cuda")
    h = torch.empty(0, 16, 32, dtype=torch.bfloat16, device="cuda")
    V = torch.randn(16, 32, device="cuda").to(torch.bfloat16)
    dV = torch.full((16, 32), float("nan"), device="cuda")
    binding.dsc_headwise_gen_fwd(h, V, x, torch.empty_like(x), W=4)
    binding.dsc_headwise_gen_bwd(h, V, x, x, torch.empty_like(x), torch.empty_like(h), dV, None, W=4)
    torch.cuda.synchronize()
    assert torch.equal(dV, torch.zeros_like(dV))


# (workload, hidden width K)
GEN_FULL = [(4, 2048), (2, 768)]


@pytest.mark.parametrize("cfg,K", GEN_FULL, ids=[f"cfg{c[0]}-K{c[1]}" for c in GEN_FULL])
def test_generated_headwise_full_size(cfg, K):
    """The head-wise workloads with filters generated from a hidden state of
    width K: every output element written; token windows (tile edges, the
    ends) of y, dx, dh and blocks of groups of dV against the oracle."""
    wl = inputs.WORKLOADS[cfg]
    inp = inputs.generator_inputs(wl, K)
    N, D, W, H = wl.N, wl.D, wl.W, wl.H
    G = D // H
    say(f"[generator] {wl.name}: B={wl.B} T={wl.T} D={D} W={W} H={H} K={K}")
    y, dx, dh, dV = _run(inp, W, H, wl.residual)
    for name, g in (("y", y), ("dx", dx), ("dh", dh), ("dV", dV)):
        assert not torch.isnan(g.t).any().item(), f"{name}: unwritten elements"
    x64, g64, V64, h64 = (to_f64(inp[k]) for k in ("x", "dy", "V", "h"))
    kw = dict(W=W, cu_seqlens=inp["cu_seqlens"], residual=wl.residual)
    tol = TOL["bf16"]
    step = 128 - (W - 1)
    for lo, hi in [(0, 40), (step - 5, step + 5), (4090, 4110), (N // 2 - 7, N // 2 + 17), (N - 40, N)]:
        say(f"  rows [{lo},{hi})")
        assert_close("y", to_f64(y.t.reshape(N, D)[lo:hi]),
                     oracle.headwise_gen_fwd(h64, V64, x64, rows=(lo, hi), **kw), tol)
        rdx, rdh, _ = oracle.headwise_gen_bwd(h64, V64, x64, g64, rows=(lo, hi), groups=(0, 0), **kw)
        assert_close("dx", to_f64(dx.t.reshape(N, D)[lo:hi]), rdx, tol)
        assert_close("dh", to_f64(dh.t.reshape(N, K)[lo:hi]), rdh, tol)
    dVf = dV.host()
    for g0, g1 in [(0, 4), (G // 2 - 2, G // 2 + 2), (G - 4, G)]:
        say(f"  dV groups [{g0},{g1})")
        _, _, rdV = oracle.headwise_gen_bwd(h64, V64, x64, g64, rows=(0, 0), groups=(g0, g1), **kw)
        assert_close("dV", dVf[g0 * W:g1 * W], rdV, tol)
