"""Tensors beyond 4 GiB (GPU): B=256 T=4096 D=2304 W=4, 1,048,576 tokens, so
each bf16 activation holds 2.4e9 elements (4.8 GB) and its element and byte
offsets pass 2^31 and 2^32.  Inputs are counter-based (their values depend on
the element index alone) and are drawn on the GPU; the oracle sees host
windows of them (tests/large_util.py, checked on the CPU against whole
tensors): token windows at the start, across the 2^31-byte and 2^32-byte
offsets, across a sequence start and at the end, and channel slices for the
sums over every token (dU, dc).  Every output starts as NaN and is checked
on the device to have been written in full."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import large_util as lu
from gpu_util import TOL, assert_close, say
from input_dependent_short_amd import binding, inputs
from input_dependent_short_amd.inputs import to_f64

pytestmark = pytest.mark.gpu

B, T, D, W = 256, 4096, 2304, 4
N = B * T
DT = "bf16"
ROWS = [(0, 16), (2**30 // D - 6, 2**30 // D + 10), (2**31 // D - 8, 2**31 // D + 8),
        (228 * T - 8, 228 * T + 8), (N - 16, N)]
CHANNELS = [(0, 8), (D - 8, D)]


def _seeds(base: int) -> dict:
    return {k: inputs.seed_for(base, i) for i, k in enumerate(("x", "w", "dy", "z", "U", "c"))}


def _gpu(seed: int, std: float, shape) -> torch.Tensor:
    return inputs.counter_tensor(shape, seed, std, DT, "cuda")


def _nan(shape, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def _rows(t: torch.Tensor, lo: int, hi: int) -> np.ndarray:
    return to_f64(t.view(N, -1)[lo:hi])


def _written(**outs) -> None:
    """Every element of each full-size output was written (checked on the device)."""
    for name, t in outs.items():
        bad = int(torch.isnan(t).sum().item())
        say(f"  {name}: all {t.numel()} elements written" if not bad else f"  {name}: {bad} unwritten")
        assert bad == 0, f"{name}: {bad} elements not written"


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _packed(seed: int):
    """Packed sequences of 256..4096 tokens (the 2B varlen recipe), and extra
    windows across the sequence starts nearest the 2^31- and 2^32-byte offsets."""
    cu = inputs.packed_cu_seqlens(B, T, 256, 4096, seed)
    extra = []
    for n in (2**30 // D, 2**31 // D):
        c = int(cu[np.searchsorted(cu, n)])
        extra.append((c - 8, c + 8))
    return cu, ROWS + extra


@pytest.mark.parametrize("varlen", [False, True], ids=["rows", "packed"])
def test_headwise_beyond_4gib(varlen):
    H = 64
    G = D // H
    s = _seeds(901)
    cu_np, rows = _packed(906) if varlen else (None, ROWS)
    cu = None if cu_np is None else torch.from_numpy(cu_np).cuda()
    say(f"[large headwise] B={B} T={T} D={D} H={H}: {N * D * 2 / 1e9:.2f} GB per activation, "
        f"{'packed' if varlen else 'rows'}")
    x, dy = _gpu(s["x"], 1.0, (B, T, D)), _gpu(s["dy"], 1.0, (B, T, D))
    w = _gpu(s["w"], 1.0 / np.sqrt(W), (B, T, G, W))
    y, dx, dw = _nan((B, T, D)), _nan((B, T, D)), _nan((B, T, G, W))
    binding.dsc_headwise_fwd(x, w, y, cu_seqlens=cu, residual=True)
    binding.dsc_headwise_bwd(x, w, dy, dx, dw, cu_seqlens=cu, residual=True)
    torch.cuda.synchronize()
    _written(y=y, dx=dx, dw=dw)
    tol = TOL[DT]
    for lo, hi in rows:
        say(f"  rows [{lo},{hi})")
        ry, rdx, rdw = lu.headwise_rows(s, N, T, D, G, W, lo, hi, True, DT, cu_np)
        assert_close("y", _rows(y, lo, hi), ry, tol)
        assert_close("dx", _rows(dx, lo, hi), rdx, tol)
        assert_close("dw", _rows(dw, lo, hi).reshape(hi - lo, G, W), rdw, tol)
    del x, dy, w, y, dx, dw
    _free()


@pytest.mark.parametrize("varlen", [False, True], ids=["rows", "packed"])
def test_lowrank_beyond_4gib(varlen):
    R = 32
    s = _seeds(902)
    cu_np, rows = _packed(907) if varlen else (None, ROWS)
    cu = None if cu_np is None else torch.from_numpy(cu_np).cuda()
    say(f"[large lowrank] B={B} T={T} D={D} R={R}, {'packed' if varlen else 'rows'}")
    x, dy = _gpu(s["x"], 1.0, (B, T, D)), _gpu(s["dy"], 1.0, (B, T, D))
    z = _gpu(s["z"], 1.0, (B, T, R))
    U = _gpu(s["U"], 1.0 / np.sqrt(R * W), (R, D * W))
    y, dx, dz = _nan((B, T, D)), _nan((B, T, D)), _nan((B, T, R))
    dU = _nan((R, D * W), torch.float32)
    nws = binding.dsc_lowrank_bwd_workspace_size(x.dtype, B, T, D, W, R)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    binding.dsc_lowrank_fwd(x, z, U, y, W=W, cu_seqlens=cu)
    binding.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws, W=W, cu_seqlens=cu)
    torch.cuda.synchronize()
    _written(y=y, dx=dx, dz=dz, dU=dU)
    tol = TOL[DT]
    for lo, hi in rows:
        say(f"  rows [{lo},{hi})")
        ry, rdx, rdz = lu.lowrank_rows(s, N, T, D, R, W, lo, hi, False, DT, cu_np)
        assert_close("y", _rows(y, lo, hi), ry, tol)
        assert_close("dx", _rows(dx, lo, hi), rdx, tol)
        assert_close("dz", _rows(dz, lo, hi), rdz, tol)
    dU3 = dU.cpu().double().numpy().reshape(R, D, W)
    for c0, c1 in CHANNELS:
        say(f"  dU channels [{c0},{c1})")
        assert_close("dU", dU3[:, c0:c1].reshape(R, -1), lu.lowrank_dU(s, B, T, D, R, W, c0, c1, DT, cu_np), tol)
    del x, dy, z, U, y, dx, dz, dU, ws
    _free()


def test_static_beyond_4gib():
    s = _seeds(903)
    say(f"[large static] B={B} T={T} D={D}")
    x, dy = _gpu(s["x"], 1.0, (B, T, D)), _gpu(s["dy"], 1.0, (B, T, D))
    c = _gpu(s["c"], 1.0 / np.sqrt(W), (D, W))
    y, dx = _nan((B, T, D)), _nan((B, T, D))
    dc = _nan((D, W), torch.float32)
    binding.dsc_static_fwd(x, c, y, residual=True)
    binding.dsc_static_bwd(x, c, dy, dx, dc, residual=True)
    torch.cuda.synchronize()
    _written(y=y, dx=dx, dc=dc)
    tol = TOL[DT]
    for lo, hi in ROWS:
        say(f"  rows [{lo},{hi})")
        ry, rdx = lu.static_rows(s, N, T, D, W, lo, hi, True, DT)
        assert_close("y", _rows(y, lo, hi), ry, tol)
        assert_close("dx", _rows(dx, lo, hi), rdx, tol)
    dcn = dc.cpu().double().numpy()
    for c0, c1 in CHANNELS:
        say(f"  dc channels [{c0},{c1})")
        assert_close("dc", dcn[c0:c1], lu.static_dc(s, B, T, D, W, c0, c1, DT), tol)
    del x, dy, c, y, dx, dc
    _free()


def _seq_rows(seed: int, std: float, tail: tuple, lo: int, hi: int) -> np.ndarray:
    return lu.rows_of(seed, std, DT, tail, lo, hi)


@pytest.mark.parametrize("kind", ["headwise", "lowrank"])
def test_decode_at_the_batch_limit(kind):
    """One decoding step for the largest batch the ABI takes at D = 2304
    (B*D < 2^31: 932,067 sequences): the (B, W-1, D) state holds 6.4e9 elements,
    so its offsets pass 2^32.  Sequence windows at the start, across the 2^31-
    byte offset of x and y, across the 2^31- and 2^32-element offsets of the
    state, and at the end (x and y end just below 2^32 bytes); y and the
    updated state against the oracle."""
    import oracle
    H, R = 64, 32
    G = D // H
    Bd = (2**31 - 1) // D
    s = _seeds(904 if kind == "headwise" else 905)
    say(f"[large decode {kind}] B={Bd} D={D} W={W}: state {Bd * (W - 1) * D * 2 / 1e9:.1f} GB")
    x = _gpu(s["x"], 1.0, (Bd, D))
    st = _gpu(s["c"], 1.0, (Bd, W - 1, D))
    y = _nan((Bd, D))
    if kind == "headwise":
        w = _gpu(s["w"], 1.0 / np.sqrt(W), (Bd, G, W))
        binding.dsc_headwise_decode(x, w, st, y, residual=True)
    else:
        z = _gpu(s["z"], 1.0, (Bd, R))
        U = _gpu(s["U"], 1.0 / np.sqrt(R * W), (R, D * W))
        binding.dsc_lowrank_decode(x, z, U, st, y, W=W)
    torch.cuda.synchronize()
    _written(y=y)
    per = (W - 1) * D
    wins = [(0, 8), (2**30 // D - 4, 2**30 // D + 4), (2**31 // per - 4, 2**31 // per + 4),
            (2**32 // per - 4, 2**32 // per + 4), (Bd - 8, Bd)]
    U64 = _seq_rows(s["U"], 1.0 / np.sqrt(R * W), (D * W,), 0, R) if kind == "lowrank" else None
    tol = TOL[DT]
    for lo, hi in wins:
        say(f"  sequences [{lo},{hi})")
        xw = _seq_rows(s["x"], 1.0, (D,), lo, hi)
        sw = _seq_rows(s["c"], 1.0, (W - 1, D), lo, hi)
        if kind == "headwise":
            ry, rst = oracle.headwise_decode(xw, _seq_rows(s["w"], 1.0 / np.sqrt(W), (G, W), lo, hi), sw,
                                             residual=True)
        else:
            ry, rst = oracle.lowrank_decode(xw, _seq_rows(s["z"], 1.0, (R,), lo, hi), U64, sw, W)
        assert_close("y", to_f64(y[lo:hi]), ry, tol)
        assert np.array_equal(to_f64(st[lo:hi]), rst), "state rows differ from the oracle's shift"
    del x, st, y
    _free()
