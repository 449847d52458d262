"""GPU parity of the head-wise and low-rank layers fused with the rotary
position embedding of the query and key channels, and of its cos / sin table,
through the C ABI against the fp64 oracle.

The table is compared entry by entry with the oracle's double-precision table
rounded to fp32 (at most one fp32 ulp apart: both sides take cos / sin in
double precision and round once).  The fused layer's y, dx and dw are compared
element by element at small shapes and on sampled token windows at the QKV
~150M shape (B=8 T=2048 D=2304 W=4, heads of 64, query + key = 1536
channels), with the normwise tolerance of the layer itself (1e-5 fp32, 2e-2
bf16).  The low-rank layer's y, dx, dz and dU are compared the same way at
small shapes (every kernel family) and at the QKV ~150M (R = 32, heads of 64)
and QKV ~2B (R = 64, packed sequences, heads of 128) workloads.
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


def _table(max_pos: int, hd: int, base: float) -> torch.Tensor:
    t = Guarded((max_pos, hd // 2, 2), torch.float32)
    binding.dsc_rope_table(t.t, base=base)
    torch.cuda.synchronize()
    t.check_guards("table")
    return t.t


@pytest.mark.parametrize("max_pos,hd,base", [(2048, 64, 10000.0), (37, 8, 500.0), (16384, 128, 1e6), (5, 2, 3.0)])
def test_rope_table(max_pos, hd, base):
    say(f"[rope] table max_pos={max_pos} head_dim={hd} base={base}")
    got = _table(max_pos, hd, base).cpu().numpy().astype(np.float64)
    want = oracle.rope_table(max_pos, hd, base).astype(np.float32)
    ulp = np.spacing(np.abs(want)).astype(np.float64)
    diff = np.abs(got - want.astype(np.float64))
    assert np.all(diff <= ulp), f"max difference {np.max(diff / ulp):.2f} fp32 ulp"


def _run(inp, res, rot, hd, table):
    x, w, dy = inp["x"].cuda(), inp["w"].cuda(), inp["dy"].cuda()
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    y, dx, dw = Guarded(x.shape, x.dtype), Guarded(x.shape, x.dtype), Guarded(w.shape, w.dtype)
    kw = dict(rot=rot, head_dim=hd, table=table, cu_seqlens=cu, residual=res)
    binding.dsc_headwise_rope_fwd(x, w, y.t, **kw)
    binding.dsc_headwise_rope_bwd(x, w, dy, dx.t, dw.t, **kw)
    torch.cuda.synchronize()
    for name, g in (("y", y), ("dx", dx), ("dw", dw)):
        g.check_guards(name)
    return y, dx, dw


# (dtype, B, T, D, W, H, head_dim, rot, residual, segment-length range or None)
RP_CASES = [
    ("fp32", 2, 37, 96, 4, 4, 16, 64, True, None),
    ("fp32", 1, 50, 64, 3, 1, 8, 32, False, (1, 9)),
    ("fp32", 2, 33, 32, 1, 4, 4, 32, True, (1, 5)),      # W = 1, every channel rotated
    ("bf16", 2, 100, 192, 4, 64, 64, 128, True, None),    # query, key, value heads of 64
    ("bf16", 1, 300, 768, 4, 64, 64, 512, True, (1, 40)),
    ("bf16", 3, 19, 48, 2, 8, 16, 32, False, None),
    ("bf16", 1, 130, 256, 8, 16, 32, 256, True, (1, 40)),
    ("bf16", 2, 66, 512, 7, 2, 64, 256, False, None),     # four filter groups per 16-byte chunk
    ("bf16", 4, 65, 2304, 4, 64, 64, 1536, True, None),   # the QKV layout at a short length
    ("bf16", 1, 1, 16, 3, 8, 8, 8, False, None),          # one token
    # any H: groups across 16-byte chunks (3, 6), lane groups padded to a power of two (24, 48, 96)
    ("bf16", 2, 60, 96, 4, 3, 16, 64, True, (1, 20)),
    ("bf16", 1, 70, 192, 4, 6, 32, 128, False, None),
    ("bf16", 2, 50, 192, 4, 24, 32, 128, True, (1, 30)),
    ("bf16", 1, 90, 384, 4, 48, 64, 256, True, None),
    ("bf16", 1, 40, 768, 3, 96, 64, 512, False, (1, 25)),
    ("fp32", 1, 30, 48, 4, 3, 8, 32, True, None),
]


def _ids(cases):
    return [f"rope-{c[0]}-B{c[1]}T{c[2]}D{c[3]}W{c[4]}H{c[5]}-hd{c[6]}rot{c[7]}-res{int(c[8])}-"
            f"{'varlen' if c[9] else 'rows'}" for c in cases]


@pytest.mark.parametrize("case", RP_CASES, ids=_ids(RP_CASES))
def test_headwise_rope_small(case):
    dt, B, T, D, W, H, hd, rot, res, seg = case
    wl, inp = inputs.small("headwise", B, T, D, W, H=H, dtype=dt, residual=res, varlen=seg is not None,
                           seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    cu = inp["cu_seqlens"]
    base = 10000.0 if hd >= 32 else 100.0
    max_pos = B * T if cu is not None else T
    say(f"[rope] {wl.name} hd={hd} rot={rot} residual={res} segments={cu}")
    table = _table(max_pos, hd, base)
    y, dx, dw = _run(inp, res, rot, hd, table)
    x64, w64, g64 = (to_f64(inp[k]) for k in ("x", "w", "dy"))
    kw = dict(rot=rot, head_dim=hd, base=base, cu_seqlens=cu, residual=res)
    ry = oracle.headwise_rope_fwd(x64, w64, **kw)
    rdx, rdw = oracle.headwise_rope_bwd(x64, w64, g64, **kw)
    tol = TOL[dt]
    assert_close("y", y.host(), ry, tol)
    assert_close("dx", dx.host(), rdx, tol)
    assert_close("dw", dw.host(), rdw, tol)
    # the backward has no atomics: a second call gives the same bits
    _, dx2, dw2 = _run(inp, res, rot, hd, table)
    assert torch.equal(dx.t, dx2.t) and torch.equal(dw.t, dw2.t)


def test_headwise_rope_qkv_150m_full_size():
    wl = inputs.WORKLOADS[2]
    inp = inputs.make_inputs(wl)
    hd, rot = 64, 1536
    say(f"[rope] {wl.name}: B={wl.B} T={wl.T} D={wl.D} W={wl.W} H={wl.H} head_dim={hd} rot={rot}")
    table = _table(wl.T, hd, 10000.0)
    y, dx, dw = _run(inp, True, rot, hd, table)
    x64, w64, g64 = (to_f64(inp[k]) for k in ("x", "w", "dy"))
    N, D, G = wl.N, wl.D, wl.D // wl.H
    yf, dxf, dwf = y.host().reshape(N, D), dx.host().reshape(N, D), dw.host().reshape(N, G, wl.W)
    kw = dict(rot=rot, head_dim=hd, base=10000.0, residual=True)
    tol = TOL["bf16"]
    for lo, hi in [(0, 40), (2040, 2060), (N // 2 - 7, N // 2 + 17), (N - 40, N)]:
        assert_close("y", yf[lo:hi], oracle.headwise_rope_fwd(x64, w64, rows=(lo, hi), **kw), tol)
        rdx, rdw = oracle.headwise_rope_bwd(x64, w64, g64, rows=(lo, hi), **kw)
        assert_close("dx", dxf[lo:hi], rdx, tol)
        assert_close("dw", dwf[lo:hi], rdw, tol)


def test_headwise_rope_without_rotation_is_the_layer():
    """rot = 0 (no table) gives the head-wise layer's outputs bit for bit."""
    wl, inp = inputs.small("headwise", 2, 40, 256, 4, H=16, dtype="bf16", residual=True, seed=5)
    x, w, dy = inp["x"].cuda(), inp["w"].cuda(), inp["dy"].cuda()
    outs = [torch.empty_like(x) for _ in range(4)] + [torch.empty_like(w) for _ in range(2)]
    binding.dsc_headwise_rope_fwd(x, w, outs[0], rot=0, head_dim=64, table=None, residual=True)
    binding.dsc_headwise_fwd(x, w, outs[1], residual=True)
    binding.dsc_headwise_rope_bwd(x, w, dy, outs[2], outs[4], rot=0, head_dim=64, table=None, residual=True)
    binding.dsc_headwise_bwd(x, w, dy, outs[3], outs[5], residual=True)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[2], outs[3]) and torch.equal(outs[4], outs[5])


def test_headwise_rope_empty_batch():
    x = torch.empty(0, 16, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(0, 16, 4, 4, dtype=torch.bfloat16, device="cuda")
    binding.dsc_headwise_rope_fwd(x, w, torch.empty_like(x), rot=64, head_dim=16, table=None)
    binding.dsc_headwise_rope_bwd(x, w, x, torch.empty_like(x), torch.empty_like(w), rot=64, head_dim=16,
                                  table=None)
    torch.cuda.synchronize()


# ------------------------------------------------------------ low-rank layer


def _run_lr(inp, W, res, rot, hd, table):
    x, z, U, dy = (inp[k].cuda() for k in ("x", "z", "U", "dy"))
    B, T, D = x.shape
    R = z.shape[2]
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    y, dx, dz = Guarded(x.shape, x.dtype), Guarded(x.shape, x.dtype), Guarded(z.shape, z.dtype)
    dU = Guarded(U.shape, torch.float32)
    nws = binding.dsc_lowrank_bwd_workspace_size(x.dtype, B, T, D, W, R)
    ws = torch.full((max(nws, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda") if nws else None
    kw = dict(W=W, rot=rot, head_dim=hd, table=table, cu_seqlens=cu, residual=res)
    binding.dsc_lowrank_rope_fwd(x, z, U, y.t, **kw)
    binding.dsc_lowrank_rope_bwd(x, z, U, dy, dx.t, dz.t, dU.t, ws, **kw)
    torch.cuda.synchronize()
    for name, g in (("y", y), ("dx", dx), ("dz", dz), ("dU", dU)):
        g.check_guards(name)
    return y, dx, dz, dU


# (dtype, B, T, D, W, R, head_dim, rot, residual, segment-length range or None)
LRP_CASES = [
    ("fp32", 2, 37, 64, 4, 8, 16, 32, True, None),
    ("fp32", 1, 50, 48, 3, 5, 8, 48, False, (1, 9)),       # every channel rotated
    ("bf16", 2, 100, 192, 4, 32, 64, 128, True, None),     # query, key, value heads of 64
    ("bf16", 1, 300, 768, 4, 64, 64, 512, False, (1, 40)),  # R = 64: two rank tiles
    ("bf16", 1, 200, 128, 3, 20, 32, 128, True, (1, 30)),  # z rows gathered (R % 8 != 0)
    ("bf16", 1, 60, 64, 4, 100, 16, 32, False, None),      # R > 64: vector-ALU kernels
    ("bf16", 1, 90, 128, 6, 48, 32, 64, True, (1, 20)),    # wide forward, vector-ALU backward
    ("bf16", 1, 130, 256, 8, 8, 32, 256, True, (1, 40)),
    ("bf16", 2, 65, 2304, 4, 32, 64, 1536, False, None),   # the QKV ~150M layout at a short length
    ("bf16", 1, 400, 6144, 4, 64, 128, 4096, False, (1, 150)),  # the QKV ~2B layout, packed
    # two waves per 32-channel slice (33 <= R <= 64, W = 2..4): a partial last
    # slice with the rotation ending inside the block, and z rows gathered
    # (R % 4 != 0) with every channel rotated
    ("bf16", 2, 333, 136, 4, 40, 8, 64, True, (1, 50)),
    ("bf16", 1, 300, 96, 2, 45, 16, 96, False, (1, 80)),
    ("bf16", 1, 1, 16, 3, 4, 8, 8, False, None),           # one token
    # several token walks per channel pair, walks starting inside a sequence
    ("bf16", 1, 4100, 64, 3, 36, 16, 64, True, (1, 700)),
    ("bf16", 3, 1000, 128, 4, 20, 32, 128, True, (100, 900)),
    ("bf16", 2, 1500, 256, 4, 32, 64, 192, False, None),
]


def _lr_ids(cases):
    return [f"lrope-{c[0]}-B{c[1]}T{c[2]}D{c[3]}W{c[4]}R{c[5]}-hd{c[6]}rot{c[7]}-res{int(c[8])}-"
            f"{'varlen' if c[9] else 'rows'}" for c in cases]


def _check_lr(wl, inp, W, res, rot, hd, base, dt):
    cu = inp["cu_seqlens"]
    B, T = inp["x"].shape[:2]
    table = _table(B * T if cu is not None else T, hd, base)
    y, dx, dz, dU = _run_lr(inp, W, res, rot, hd, table)
    x64, z64, U64, g64 = (to_f64(inp[k]) for k in ("x", "z", "U", "dy"))
    kw = dict(rot=rot, head_dim=hd, base=base, cu_seqlens=cu, residual=res)
    ry = oracle.lowrank_rope_fwd(x64, z64, U64, W, **kw)
    rdx, rdz, rdU = oracle.lowrank_rope_bwd(x64, z64, U64, g64, W, **kw)
    tol = TOL[dt]
    assert_close("y", y.host(), ry, tol)
    assert_close("dx", dx.host(), rdx, tol)
    assert_close("dz", dz.host(), rdz, tol)
    assert_close("dU", dU.host(), rdU, tol)


@pytest.mark.parametrize("case", LRP_CASES, ids=_lr_ids(LRP_CASES))
def test_lowrank_rope_small(case):
    dt, B, T, D, W, R, hd, rot, res, seg = case
    wl, inp = inputs.small("lowrank", B, T, D, W, R=R, dtype=dt, residual=res, varlen=seg is not None,
                           seglen_range=seg or (1, 8), seed=zlib.crc32(repr(case).encode()) % 1000)
    base = 10000.0 if hd >= 32 else 100.0
    say(f"[lowrank rope] {wl.name} hd={hd} rot={rot} residual={res} segments={inp['cu_seqlens']}")
    _check_lr(wl, inp, W, res, rot, hd, base, dt)


def test_lowrank_rope_sequence_starts_at_step_edges():
    """Sequence starts at every offset around the 16-token steps: the
    position of each token restarts exactly at its sequence's first token."""
    T = 709
    starts = {0, T}
    offs = [0, 1, 2, 3, 7, 13, 14, 15]
    for j, m in enumerate(range(1, T // 16)):
        starts.add(16 * m + offs[j % len(offs)])
        if j % 5 == 0:
            starts.update({16 * m - 1, 16 * m + 1})
    wl, inp = inputs.small("lowrank", 1, T, 128, 4, R=32, dtype="bf16", residual=True, seed=23)
    inp["cu_seqlens"] = np.array(sorted(starts), dtype=np.int32)
    say(f"[lowrank rope] {wl.name} step-edge starts")
    _check_lr(wl, inp, 4, True, 64, 32, 10000.0, "bf16")


def test_lowrank_rope_without_rotation_is_the_layer():
    """rot = 0 (no table) gives the low-rank layer's outputs: y bit for bit,
    dx bit for bit, dz and dU up to the order of their fp32 atomic sums."""
    wl, inp = inputs.small("lowrank", 2, 70, 256, 4, R=32, dtype="bf16", residual=True, seed=6)
    x, z, U, dy = (inp[k].cuda() for k in ("x", "z", "U", "dy"))
    B, T, D = x.shape
    ws = torch.empty(binding.dsc_lowrank_bwd_workspace_size(x.dtype, B, T, D, 4, 32) // 4, device="cuda")
    y1, y2, dx1, dx2 = (torch.empty_like(x) for _ in range(4))
    dz1, dz2 = torch.empty_like(z), torch.empty_like(z)
    dU1, dU2 = (torch.empty(U.shape, dtype=torch.float32, device="cuda") for _ in range(2))
    binding.dsc_lowrank_rope_fwd(x, z, U, y1, W=4, rot=0, head_dim=64, table=None, residual=True)
    binding.dsc_lowrank_fwd(x, z, U, y2, W=4, residual=True)
    binding.dsc_lowrank_rope_bwd(x, z, U, dy, dx1, dz1, dU1, ws, W=4, rot=0, head_dim=64, table=None, residual=True)
    binding.dsc_lowrank_bwd(x, z, U, dy, dx2, dz2, dU2, ws, W=4, residual=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(dx1, dx2)
    assert torch.allclose(dz1.float(), dz2.float(), rtol=1e-2, atol=1e-2)
    assert torch.allclose(dU1, dU2, rtol=1e-4, atol=1e-4)


def test_lowrank_rope_empty_batch():
    x = torch.empty(0, 16, 64, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(0, 16, 8, dtype=torch.bfloat16, device="cuda")
    U = torch.randn(8, 64 * 4, device="cuda").to(torch.bfloat16)
    dU = torch.full((8, 256), float("nan"), device="cuda")
    binding.dsc_lowrank_rope_fwd(x, z, U, torch.empty_like(x), W=4, rot=64, head_dim=16, table=None)
    binding.dsc_lowrank_rope_bwd(x, z, U, x, torch.empty_like(x), torch.empty_like(z), dU, None, W=4, rot=64,
                                 head_dim=16, table=None)
    torch.cuda.synchronize()
    assert torch.equal(dU, torch.zeros_like(dU))  # a sum over no tokens


# (workload, head_dim, rot): the query and key channels of the QKV projections
LR_FULL = [(3, 64, 1536), (5, 128, 4096)]


@pytest.mark.parametrize("cfg,hd,rot", LR_FULL, ids=[f"cfg{c[0]}" for c in LR_FULL])
def test_lowrank_rope_full_size(cfg, hd, rot):
    """The low-rank workloads with the rotation of their query and key
    channels: every output element written, and token windows (sequence
    starts, walk boundaries, the ends) and channel blocks across the rotated
    and plain channels against the oracle."""
    wl = inputs.WORKLOADS[cfg]
    inp = inputs.make_inputs(wl)
    cu = inp["cu_seqlens"]
    N, D, W, R = wl.N, wl.D, wl.W, wl.R
    say(f"[lowrank rope] {wl.name}: B={wl.B} T={wl.T} D={D} W={W} R={R} head_dim={hd} rot={rot}")
    table = _table(N if cu is not None else wl.T, hd, 10000.0)
    y, dx, dz, dU = _run_lr(inp, W, wl.residual, rot, hd, table)
    for name, g in (("y", y), ("dx", dx), ("dz", dz), ("dU", dU)):
        assert not torch.isnan(g.t).any().item(), f"{name}: unwritten elements"
    x64, z64, U64, g64 = (to_f64(inp[k]) for k in ("x", "z", "U", "dy"))
    kw = dict(rot=rot, head_dim=hd, base=10000.0, cu_seqlens=cu, residual=wl.residual)
    tol = TOL[wl.dtype]
    wins = [(0, 40), (4090, 4110), (N // 2 - 7, N // 2 + 17), (N - 40, N)]
    if cu is not None:
        s = int(cu[len(cu) // 2])
        wins.append((max(0, s - 20), min(N, s + 20)))
    for lo, hi in wins:
        say(f"  rows [{lo},{hi})")
        yr = to_f64(y.t.reshape(N, D)[lo:hi])
        assert_close("y", yr, oracle.lowrank_rope_fwd(x64, z64, U64, W, rows=(lo, hi), **kw).reshape(hi - lo, D),
                     tol)
        rdx, rdz, _ = oracle.lowrank_rope_bwd(x64, z64, U64, g64, W, rows=(lo, hi), channels=(0, 0), **kw)
        assert_close("dx", to_f64(dx.t.reshape(N, D)[lo:hi]), rdx.reshape(hi - lo, D), tol)
        assert_close("dz", to_f64(dz.t.reshape(N, R)[lo:hi]), rdz.reshape(hi - lo, R), tol)
    dUf = to_f64(dU.t).reshape(R, D, W)
    for c0, c1 in [(0, 64), (rot - 64, rot + 64), (D - 64, D)]:
        say(f"  dU channels [{c0},{c1})")
        _, _, part = oracle.lowrank_rope_bwd(x64, z64, U64, g64, W, rows=(0, 0), channels=(c0, c1), **kw)
        assert_close("dU", dUf[:, c0:c1], part.reshape(R, c1 - c0, W), tol)


# ------------------------------------------------------------ decoding

# (dtype, B sequences, D, W, H, head_dim, rot)
RD_CASES = [("bf16", 7, 2304, 4, 64, 64, 1536), ("bf16", 33, 256, 3, 2, 32, 128), ("fp32", 4, 96, 4, 1, 16, 64),
            ("bf16", 5, 128, 1, 16, 8, 128)]


@pytest.mark.parametrize("case", RD_CASES, ids=[f"rdec-{c[0]}-B{c[1]}D{c[2]}W{c[3]}H{c[4]}-hd{c[5]}rot{c[6]}"
                                                for c in RD_CASES])
def test_headwise_rope_decode_steps(case):
    dt, B, D, W, H, hd, rot = case
    rng = np.random.default_rng(B * 100 + D + hd)
    tdt = inputs.DTYPES[dt]

    def dev(a):
        return torch.from_numpy(a.astype(np.float32)).to(tdt).cuda()

    max_pos = 64
    table = _table(max_pos, hd, 10000.0)
    st0 = dev(rng.standard_normal((B, W - 1, D)))
    state, ref_state = st0.clone(), to_f64(st0)
    pos = rng.integers(0, max_pos - 5, size=B).astype(np.int32)
    say(f"[rope decode] {dt} B={B} D={D} W={W} H={H} hd={hd} rot={rot}")
    for t in range(5):
        x = dev(rng.standard_normal((B, D)))
        w = dev(rng.standard_normal((B, D // H, W)) / np.sqrt(W))
        y = Guarded((B, D), tdt)
        p = torch.from_numpy(pos + t).cuda()
        binding.dsc_headwise_rope_decode(x, w, state, y.t, p, rot=rot, head_dim=hd, table=table,
                                         residual=bool(t % 2))
        torch.cuda.synchronize()
        y.check_guards("y")
        ry, ref_state = oracle.headwise_rope_decode(to_f64(x), to_f64(w), ref_state, pos + t, rot=rot, head_dim=hd,
                                                    base=10000.0, residual=bool(t % 2))
        assert_close("y", y.host(), ry, TOL[dt])
        assert np.array_equal(to_f64(state), ref_state), f"state after step {t}"


def test_prefill_then_rotated_decode():
    """Packed prefill through the fused forward, the state it hands over, then
    rotated decoding steps at positions len + j: every output equals the fused
    forward over the whole extended sequence."""
    D, W, H, hd, rot = 256, 4, 16, 32, 128
    wl, inp = inputs.small("headwise", 1, 300, D, W, H=H, dtype="bf16", residual=True, varlen=True,
                           seglen_range=(1, 40), seed=17)
    cu = inp["cu_seqlens"]
    S = len(cu) - 1
    lens = np.diff(cu).astype(np.int32)
    table = _table(400, hd, 10000.0)
    x, w = inp["x"].cuda(), inp["w"].cuda()
    cu_d = torch.from_numpy(cu).cuda()
    say(f"[rope decode] prefill of {S} sequences, then 3 rotated steps")
    y = torch.empty_like(x)
    binding.dsc_headwise_rope_fwd(x, w, y, rot=rot, head_dim=hd, table=table, cu_seqlens=cu_d, residual=True)
    state = torch.empty(S, W - 1, D, dtype=x.dtype, device="cuda")
    binding.dsc_state_from_prefill(x, state, W=W, cu_seqlens=cu_d)
    x64, w64 = to_f64(inp["x"]), to_f64(inp["w"])
    assert_close("prefill y", to_f64(y), oracle.headwise_rope_fwd(x64, w64, rot=rot, head_dim=hd, cu_seqlens=cu,
                                                                   residual=True), TOL["bf16"])
    rng = np.random.default_rng(8)
    seqs = [(x64[0, a:b], w64[0, a:b]) for a, b in zip(cu[:-1], cu[1:])]
    for j in range(3):
        xt = torch.from_numpy(rng.standard_normal((S, D)).astype(np.float32)).to(torch.bfloat16).cuda()
        wt = torch.from_numpy((rng.standard_normal((S, D // H, W)) / 2).astype(np.float32)).to(torch.bfloat16).cuda()
        yt = torch.empty_like(xt)
        binding.dsc_headwise_rope_decode(xt, wt, state, yt, torch.from_numpy(lens + j).cuda(), rot=rot, head_dim=hd,
                                         table=table, residual=True)
        torch.cuda.synchronize()
        xt64, wt64 = to_f64(xt), to_f64(wt)
        seqs = [(np.vstack([sx, xt64[s][None]]), np.concatenate([sw, wt64[s][None]])) for s, (sx, sw) in enumerate(seqs)]
        want = np.stack([oracle.headwise_rope_fwd(sx[None], sw[None], rot=rot, head_dim=hd, residual=True)[0, -1]
                         for sx, sw in seqs])
        assert_close("y", to_f64(yt), want, TOL["bf16"])


def test_rotated_decode_position_outside_the_table():
    """A position with no table row gives NaN in that sequence's rotated
    channels only; the other channels, the other sequences and the state are
    those of the plain step."""
    B, D, W, H, hd, rot = 4, 128, 4, 16, 32, 64
    g = torch.Generator().manual_seed(4)
    x = torch.randn(B, D, generator=g).to(torch.bfloat16).cuda()
    w = torch.randn(B, D // H, W, generator=g).to(torch.bfloat16).cuda()
    st0 = torch.randn(B, W - 1, D, generator=g).to(torch.bfloat16).cuda()
    table = _table(10, hd, 10000.0)
    pos = torch.tensor([-1, 10, 3, 9], dtype=torch.int32).cuda()
    s1, s2 = st0.clone(), st0.clone()
    y1, y2 = torch.empty_like(x), torch.empty_like(x)
    binding.dsc_headwise_rope_decode(x, w, s1, y1, pos, rot=rot, head_dim=hd, table=table)
    binding.dsc_headwise_decode(x, w, s2, y2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.isnan(y1[:2, :rot]).all() and not torch.isnan(y1[2:]).any()
    assert torch.equal(y1[:, rot:], y2[:, rot:])
    want = oracle.rope_at(to_f64(y2[2:]), [3, 9], rot=rot, head_dim=hd)
    assert_close("in-range rows", to_f64(y1[2:]), want, TOL["bf16"])
