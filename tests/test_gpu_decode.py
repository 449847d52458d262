"""GPU parity of decoding (one token per sequence, rolling state) and of the
state hand-off after a prefill, through the C ABI, against the fp64 oracle.

Each test decodes several steps in a row on the GPU, feeding back the state
the kernels wrote, and compares every step's output and the final state with
the oracle's step (which its pins tie to the forward pass).  The state holds
inputs, so it is compared bit for bit; y uses the usual normwise tolerance
(1e-5 fp32, 2e-2 bf16).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, Guarded, assert_close, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu

STEPS = 5


def _tensor(a: np.ndarray, dt: str) -> torch.Tensor:
    return torch.from_numpy(a.astype(np.float32)).to(inputs.DTYPES[dt]).cuda()


# (dtype, B sequences, D, W, H)
HW_DEC = [("bf16", 1, 64, 4, 64), ("bf16", 7, 2304, 4, 64), ("bf16", 33, 256, 3, 2), ("bf16", 5, 128, 8, 16),
          ("bf16", 3, 64, 1, 8), ("fp32", 4, 96, 4, 1), ("fp32", 2, 32, 6, 8),
          # any H with D % H == 0, groups across 16-byte chunks or of several chunks
          ("bf16", 6, 96, 4, 3), ("bf16", 3, 96, 4, 6), ("bf16", 4, 192, 4, 24), ("bf16", 2, 480, 3, 48),
          ("bf16", 5, 768, 4, 96), ("fp32", 3, 60, 5, 3)]


@pytest.mark.parametrize("case", HW_DEC, ids=[f"hw-{c[0]}-B{c[1]}D{c[2]}W{c[3]}H{c[4]}" for c in HW_DEC])
def test_headwise_decode_steps(case):
    dt, B, D, W, H = case
    rng = np.random.default_rng(B * 1000 + D + W)
    xs = [_tensor(rng.standard_normal((B, D)), dt) for _ in range(STEPS)]
    ws = [_tensor(rng.standard_normal((B, D // H, W)) / np.sqrt(W), dt) for _ in range(STEPS)]
    st0 = _tensor(rng.standard_normal((B, W - 1, D)), dt)  # a state from earlier tokens
    state = st0.clone()
    ref_state = to_f64(st0)
    say(f"[decode] head-wise {dt} B={B} D={D} W={W} H={H}")
    for t in range(STEPS):
        y = Guarded((B, D), xs[t].dtype)
        binding.dsc_headwise_decode(xs[t], ws[t], state, y.t, residual=bool(t % 2))
        torch.cuda.synchronize()
        y.check_guards("y")
        ry, ref_state = oracle.headwise_decode(to_f64(xs[t]), to_f64(ws[t]), ref_state, residual=bool(t % 2))
        assert_close("y", y.host(), ry, TOL[dt])
        assert np.array_equal(to_f64(state), ref_state), f"state after step {t}"


# (dtype, B sequences, D, W, R)
LR_DEC = [("bf16", 1, 64, 4, 32), ("bf16", 8, 2304, 4, 32), ("bf16", 70, 512, 4, 64), ("bf16", 3, 128, 2, 5),
          ("bf16", 2, 256, 8, 128), ("fp32", 4, 64, 4, 16), ("fp32", 1, 32, 1, 3), ("bf16", 5, 256, 3, 16)]


@pytest.mark.parametrize("case", LR_DEC, ids=[f"lr-{c[0]}-B{c[1]}D{c[2]}W{c[3]}R{c[4]}" for c in LR_DEC])
def test_lowrank_decode_steps(case):
    dt, B, D, W, R = case
    rng = np.random.default_rng(B * 1000 + D + R)
    U = _tensor(rng.standard_normal((R, D * W)) / np.sqrt(R * W), dt)
    xs = [_tensor(rng.standard_normal((B, D)), dt) for _ in range(STEPS)]
    zs = [_tensor(rng.standard_normal((B, R)), dt) for _ in range(STEPS)]
    state = torch.zeros(B, W - 1, D, dtype=inputs.DTYPES[dt], device="cuda")
    ref_state = np.zeros((B, W - 1, D))
    say(f"[decode] low-rank {dt} B={B} D={D} W={W} R={R}")
    for t in range(STEPS):
        y = Guarded((B, D), xs[t].dtype)
        binding.dsc_lowrank_decode(xs[t], zs[t], U, state, y.t, W=W, residual=bool(t % 2))
        torch.cuda.synchronize()
        y.check_guards("y")
        ry, ref_state = oracle.lowrank_decode(to_f64(xs[t]), to_f64(zs[t]), to_f64(U), ref_state, W,
                                              residual=bool(t % 2))
        assert_close("y", y.host(), ry, TOL[dt])
        assert np.array_equal(to_f64(state), ref_state), f"state after step {t}"


@pytest.mark.parametrize("dt,W", [("bf16", 4), ("bf16", 8), ("fp32", 3)])
def test_prefill_then_decode(dt, W):
    """Packed prefill (sequences of 1..40 tokens), the state it hands over, then
    decoding steps: every output equals the forward over the whole sequence."""
    D, H = 256, 16
    wl, inp = inputs.small("headwise", 1, 300, D, W, H=H, dtype=dt, residual=True, varlen=True,
                           seglen_range=(1, 40), seed=W)
    cu = inp["cu_seqlens"]
    S = len(cu) - 1
    x, w = inp["x"].cuda(), inp["w"].cuda()
    say(f"[decode] prefill of {S} sequences {cu.tolist()[:8]}... W={W} {dt}")
    y = torch.empty_like(x)
    cu_d = torch.from_numpy(cu).cuda()
    binding.dsc_headwise_fwd(x, w, y, cu_seqlens=cu_d, residual=True)
    state = Guarded((S, W - 1, D), x.dtype)
    binding.dsc_state_from_prefill(x, state.t, W=W, cu_seqlens=cu_d)
    torch.cuda.synchronize()
    state.check_guards("state")
    x64, w64 = to_f64(inp["x"]), to_f64(inp["w"])
    assert np.array_equal(state.host(), oracle.state_from_prefill(x64, W, cu_seqlens=cu)), "prefill state"
    # decode steps for every sequence at once, checked against the forward of each extended sequence
    rng = np.random.default_rng(7)
    st = state.t.clone()
    seqs = [(x64[0, a:b], w64[0, a:b]) for a, b in zip(cu[:-1], cu[1:])]
    for j in range(3):
        xt = _tensor(rng.standard_normal((S, D)), dt)
        wt = _tensor(rng.standard_normal((S, D // H, W)) / np.sqrt(W), dt)
        yt = torch.empty_like(xt)
        binding.dsc_headwise_decode(xt, wt, st, yt, residual=True)
        torch.cuda.synchronize()
        xt64, wt64 = to_f64(xt), to_f64(wt)
        seqs = [(np.vstack([sx, xt64[s][None]]), np.concatenate([sw, wt64[s][None]])) for s, (sx, sw) in enumerate(seqs)]
        want = np.stack([oracle.headwise_fwd(sx[None], sw[None], residual=True)[0, -1] for sx, sw in seqs])
        assert_close("y", to_f64(yt), want, TOL[dt])


def test_decode_empty_and_width_one():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(0, 8, 4, dtype=torch.bfloat16, device="cuda")
    binding.dsc_headwise_decode(x, w, torch.empty(0, 3, 64, dtype=torch.bfloat16, device="cuda"), x)
    # W = 1: no state; y = (rho + w) x
    xb = torch.randn(3, 64, device="cuda").to(torch.bfloat16)
    w1 = torch.randn(3, 8, 1, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(xb)
    binding.lib().dsc_headwise_decode(binding._stream(None), 1, 3, 64, 1, 8, binding._ptr(xb), binding._ptr(w1),
                                      None, 1, binding._ptr(y))
    torch.cuda.synchronize()
    want = (1.0 + to_f64(w1)[:, :, 0].repeat(8, axis=1)) * to_f64(xb)
    assert_close("y", to_f64(y), want, TOL["bf16"])


def test_decode_steps_replayed_as_a_graph():
    """Three decoding steps captured as one HIP graph: each replay continues the
    state and matches the same steps run eagerly (replays checked one by one,
    with eager work and synchronisation between them)."""
    rng = np.random.default_rng(3)
    B, D, W, H, R = 16, 256, 4, 16, 8
    x = _tensor(rng.standard_normal((B, D)), "bf16")
    w = _tensor(rng.standard_normal((B, D // H, W)) / 2, "bf16")
    z = _tensor(rng.standard_normal((B, R)), "bf16")
    U = _tensor(rng.standard_normal((R, D * W)) / 6, "bf16")
    st_g = torch.zeros(B, W - 1, D, dtype=torch.bfloat16, device="cuda")
    y_g = torch.empty_like(x)
    yl_g = torch.empty_like(x)
    stl_g = torch.zeros_like(st_g)

    def steps(st, y, stl, yl):
        for _ in range(3):
            binding.dsc_headwise_decode(x, w, st, y, residual=True)
            binding.dsc_lowrank_decode(x, z, U, stl, yl, W=W)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, on scratch state
        steps(torch.zeros_like(st_g), torch.empty_like(y_g), torch.zeros_like(stl_g), torch.empty_like(yl_g))
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(st_g, y_g, stl_g, yl_g)
    st_e, y_e = torch.zeros_like(st_g), torch.empty_like(y_g)
    stl_e, yl_e = torch.zeros_like(stl_g), torch.empty_like(yl_g)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        steps(st_e, y_e, stl_e, yl_e)
        torch.cuda.synchronize()
        for name, a, b in (("y", y_g, y_e), ("state", st_g, st_e), ("low-rank y", yl_g, yl_e),
                           ("low-rank state", stl_g, stl_e)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager steps"
