"""Seeded synthetic inputs for the dynamic short convolution workloads.

This module holds no arithmetic of the method: it only draws Gaussian
(or, for tensors beyond what the host should hold, counter-based uniform)
tensors, scales them, rounds them to the working dtype and builds packed
sequence offsets.  Both the GPU parity tests and the fp64 oracle consume the
same tensors it returns (the oracle receives the exact double value of every
rounded element).

Distributions: ``N(0, s^2)`` means variance ``s^2``; every fp32 draw is
rounded to the working dtype with round-to-nearest-even (torch's cast).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 20260603

DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity configuration."""
    name: str
    kind: str            # "headwise", "lowrank" or "static" (one fixed filter per channel)
    B: int
    T: int
    D: int
    W: int
    H: int = 1           # channels per shared filter (head-wise)
    R: int = 0           # rank (low-rank)
    dtype: str = "bf16"
    residual: bool = False
    varlen: bool = False
    seglen_range: tuple = (256, 4096)
    cfg: int = 0         # index used to derive seeds
    note: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.B * self.T


# The five workloads: tiny per-channel case, head-wise QKV at ~150M scale,
# low-rank QKV at ~150M scale, head-wise MLP-intermediate at ~2B scale and
# low-rank varlen QKV at ~2B scale.
WORKLOADS = {
    1: Workload("perchannel-tiny", "headwise", 1, 64, 64, 4, H=1, dtype="fp32", residual=False,
                cfg=1, note="B=1 T=64 D=64 W=4, one filter per channel, fp32"),
    2: Workload("headwise-qkv-150m", "headwise", 8, 2048, 2304, 4, H=64, dtype="bf16",
                residual=True, cfg=2, note="Q,K,V of width 768, groups of 64 channels"),
    3: Workload("lowrank-qkv-150m", "lowrank", 8, 2048, 2304, 4, R=32, dtype="bf16",
                residual=False, cfg=3, note="R=32, U (32, D*W)"),
    4: Workload("headwise-mlp-2b", "headwise", 4, 4096, 8192, 4, H=16, dtype="bf16",
                residual=True, cfg=4, note="MLP intermediate, groups of 16 channels"),
    5: Workload("lowrank-qkv-2b-varlen", "lowrank", 4, 4096, 6144, 4, R=64, dtype="bf16",
                residual=False, varlen=True, cfg=5,
                note="packed segments U{256..4096}, causal reset at each start"),
}


def seed_for(cfg: int, slot: int) -> int:
    """Seed of input slot (0 x, 1 w or z, 2 U, 3 dy, 4 segment lengths, 5 hidden
    state h, 6 generator weight V) of a workload."""
    return SEED_BASE + 10 * cfg + slot


def _normal(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(a).to(DTYPES[dtype])


def packed_cu_seqlens(B: int, T: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Segment offsets on the flattened B*T axis.

    Per row, lengths are drawn uniformly from {lo..hi} until the row's T tokens
    are filled; the last segment is cut to fit.  Segments never cross rows, so
    every row start b*T is a segment start.
    """
    rng = np.random.default_rng(seed)
    cu = [0]
    for b in range(B):
        used = 0
        while used < T:
            L = int(rng.integers(lo, hi + 1))
            L = min(L, T - used)
            used += L
            cu.append(b * T + used)
    return np.asarray(cu, dtype=np.int32)


def make_inputs(wl: Workload, *, cfg: int | None = None, seglen_seed_slot: int = 4) -> dict:
    """All inputs of a workload as CPU tensors in the workload dtype.

    Keys: x (B,T,D), dy (B,T,D), and w (B,T,D/H,W) for head-wise, z (B,T,R)
    and U (R, D*W) for low-rank, or c (D,W) for static; cu_seqlens (int32
    numpy or None).
    Scales: x, dy, z ~ N(0,1); w, c ~ N(0, 1/W); U ~ N(0, 1/(R*W)).
    """
    c = wl.cfg if cfg is None else cfg
    B, T, D, W = wl.B, wl.T, wl.D, wl.W
    out = {"x": _cast(_normal(seed_for(c, 0), (B, T, D), 1.0), wl.dtype),
           "dy": _cast(_normal(seed_for(c, 3), (B, T, D), 1.0), wl.dtype)}
    if wl.kind == "headwise":
        G = D // wl.H
        out["w"] = _cast(_normal(seed_for(c, 1), (B, T, G, W), float(1.0 / np.sqrt(W))), wl.dtype)
    elif wl.kind == "static":
        out["c"] = _cast(_normal(seed_for(c, 1), (D, W), float(1.0 / np.sqrt(W))), wl.dtype)
    else:
        R = wl.R
        out["z"] = _cast(_normal(seed_for(c, 1), (B, T, R), 1.0), wl.dtype)
        out["U"] = _cast(_normal(seed_for(c, 2), (R, D * W), float(1.0 / np.sqrt(R * W))), wl.dtype)
    out["cu_seqlens"] = (packed_cu_seqlens(B, T, *wl.seglen_range, seed_for(c, seglen_seed_slot))
                         if wl.varlen else None)
    return out


def small(kind: str, B: int, T: int, D: int, W: int, *, H: int = 1, R: int = 0,
          dtype: str = "bf16", residual: bool = False, varlen: bool = False,
          seglen_range: tuple = (1, 8), seed: int = 0) -> tuple[Workload, dict]:
    """A small ad-hoc workload (parity sweeps); seeds derive from ``seed``."""
    wl = Workload(f"{kind}-B{B}T{T}D{D}W{W}H{H}R{R}-{dtype}", kind, B, T, D, W, H=H, R=R,
                  dtype=dtype, residual=residual, varlen=varlen, seglen_range=seglen_range,
                  cfg=1000 + seed)
    return wl, make_inputs(wl)


def generator_inputs(wl: Workload, K: int, *, cfg: int | None = None) -> dict:
    """Inputs of the head-wise layer whose filters come from a hidden state:
    those of make_inputs (x, dy, cu_seqlens; the drawn w is dropped) plus the
    hidden state h (B,T,K) ~ N(0,1) and the generator's weight V (G*W, K) ~
    N(0, 1/(K*W)), so that the generated filters h V^T have the variance 1/W
    of the directly drawn ones."""
    c = wl.cfg if cfg is None else cfg
    out = make_inputs(wl, cfg=cfg)
    out.pop("w", None)
    G = wl.D // wl.H
    out["h"] = _cast(_normal(seed_for(c, 5), (wl.B, wl.T, K), 1.0), wl.dtype)
    out["V"] = _cast(_normal(seed_for(c, 6), (G * wl.W, K), float(1.0 / np.sqrt(K * wl.W))), wl.dtype)
    return out


# ---- counter-based inputs, for tensors too large to draw on the host
#
# Element i of a tensor drawn with seed s depends on (s, i) alone, so the host
# can rebuild any window of a tensor that lives only on the GPU.  The counter
# is mixed into 32 bits and passed through three rounds of xor-shift by 16 and
# multiplication by 0x45d9f3b (a well-known 32-bit integer hash); the top 24
# bits give a uniform value in [-1, 1), scaled by sqrt(3)*std so that its
# variance is std^2 like the Gaussian draws above.  Every integer step stays
# below 2^63 in int64 and the mapping to [-1, 1) is exact, so only the final
# fp32 scaling and the cast round, identically on the CPU and the GPU.

_M32 = 0xFFFFFFFF


def counter_values(seed: int, index: torch.Tensor, std: float, dtype: str) -> torch.Tensor:
    """Values of the elements at the flat positions ``index`` (int64, any device)."""
    i = index.to(torch.int64)
    x = (((i & _M32) * 0x2545F491) & _M32) + (((i >> 32) * 0x1B873593) & _M32)
    x = (x + ((seed & _M32) * 0x27D4EB2F & _M32)) & _M32
    for _ in range(3):
        x = x ^ (x >> 16)
        x = (x * 0x45D9F3B) & _M32
    x = x ^ (x >> 16)
    u = (x >> 8).to(torch.float32) * (2.0 ** -23) - 1.0
    scale = torch.tensor(float(np.sqrt(3.0) * std), dtype=torch.float32, device=u.device)
    return (u * scale).to(DTYPES[dtype])


def counter_tensor(shape, seed: int, std: float, dtype: str, device, chunk: int = 1 << 26) -> torch.Tensor:
    """A whole tensor of counter_values, filled chunk by chunk on ``device``."""
    out = torch.empty(tuple(shape), dtype=DTYPES[dtype], device=device)
    flat = out.view(-1)
    for a in range(0, flat.numel(), chunk):
        b = min(flat.numel(), a + chunk)
        flat[a:b] = counter_values(seed, torch.arange(a, b, dtype=torch.int64, device=device), std, dtype)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact double value of every element (bf16 and fp32 embed exactly in fp64)."""
    return t.detach().cpu().to(torch.float64).numpy()
