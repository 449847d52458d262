"""fp64 CPU oracle of the dynamic short convolution (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls it, and the two share no
code.  The arithmetic lives in ``dsc_oracle.c`` (plain C, double precision,
direct summation); this module only compiles it with gcc and marshals numpy
arrays through ctypes.

Definitions followed ("Dynamic Short Convolutions Improve Transformers",
gist.science technical summary, Methodology): the output is the sum over
taps k < W of w(t)_k times x_{t-k}, elementwise over channels; w(t) is either
shared by H consecutive channels (head-wise tying) or w(t) = z_t U (low rank
R); placement with residual X + conv(X).  Causal zero padding per sequence
follows the authors' thread (digg.com, "Custom Triton GPU kernels maintain
wall-clock training efficiency"): the static short convolution being
generalised is causal.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsc_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(out_path: str = LIB_PATH, extra_flags: tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           _SRC, "-o", out_path + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_abi_version.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_headwise_fwd.argtypes = [i64, i64, i64, i32, i32, p, p, p, i32, i32, i64, i64, p]
    lib.oracle_headwise_bwd.argtypes = [i64, i64, i64, i32, i32, p, p, p, p, i32, i32, i64, i64, p, p]
    lib.oracle_lowrank_fwd.argtypes = [i64, i64, i64, i32, i32, p, p, p, p, i32, i32, i64, i64, p]
    lib.oracle_lowrank_bwd.argtypes = [i64, i64, i64, i32, i32, p, p, p, p, p, i32, i32, i64, i64,
                                       p, p, i64, i64, p]
    lib.oracle_static_fwd.argtypes = [i64, i64, i64, i32, p, p, p, i32, i32, i64, i64, p]
    lib.oracle_static_bwd.argtypes = [i64, i64, i64, i32, p, p, p, p, i32, i32, i64, i64, p, p]
    lib.oracle_headwise_decode.argtypes = [i64, i64, i32, i32, p, p, p, i32, p]
    lib.oracle_lowrank_decode.argtypes = [i64, i64, i32, i32, p, p, p, p, i32, p]
    lib.oracle_state_from_prefill.argtypes = [i64, i64, i64, i32, p, p, i32, p]
    lib.oracle_rope_table.argtypes = [i64, i32, ctypes.c_double, p]
    lib.oracle_rope.argtypes = [i64, i64, i64, i64, i32, ctypes.c_double, p, i32, i32, i64, i64, p, p]
    lib.oracle_rope_at.argtypes = [i64, i64, i64, i32, ctypes.c_double, p, p, p]
    lib.oracle_generate.argtypes = [i64, i64, i64, p, p, i64, i64, p]
    lib.oracle_generate_bwd_h.argtypes = [i64, i64, p, p, i64, p]
    lib.oracle_generate_bwd_v.argtypes = [i64, i64, i64, p, p, i64, i64, p]
    for name in ("oracle_headwise_fwd", "oracle_headwise_bwd", "oracle_lowrank_fwd",
                 "oracle_lowrank_bwd", "oracle_static_fwd", "oracle_static_bwd",
                 "oracle_headwise_decode", "oracle_lowrank_decode", "oracle_state_from_prefill",
                 "oracle_rope_table", "oracle_rope", "oracle_rope_at", "oracle_generate",
                 "oracle_generate_bwd_h", "oracle_generate_bwd_v"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, 0
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    return cu, len(cu) - 1


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"{name} failed with code {rc}")


class Oracle:
    """numpy front end of one oracle library (the default one or a variant)."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    def headwise_fwd(self, x, w, *, cu_seqlens=None, residual=False, rows=None):
        """x (B,T,D), w (B,T,D/H,W) -> y (rows, D) for token rows [lo, hi) of B*T (default all)."""
        x, w = _f64(x), _f64(w)
        B, T, D = x.shape
        G, W = w.shape[2], w.shape[3]
        if G < 1 or D % G:
            raise ValueError(f"filter groups {G} do not divide D={D}")
        H = D // G
        lo, hi = rows if rows is not None else (0, B * T)
        cu, ns = _cu(cu_seqlens)
        y = np.empty((hi - lo, D))
        _check(self.lib.oracle_headwise_fwd(B, T, D, W, H, _ptr(x), _ptr(w), _ptr(cu), ns,
                                            int(bool(residual)), lo, hi, _ptr(y)), "headwise_fwd")
        return y.reshape(B, T, D) if rows is None else y

    def headwise_bwd(self, x, w, dy, *, cu_seqlens=None, residual=False, rows=None):
        """-> (dx, dw) with dx (B,T,D) and dw (B,T,G,W), or compact rows."""
        x, w, dy = _f64(x), _f64(w), _f64(dy)
        B, T, D = x.shape
        G, W = w.shape[2], w.shape[3]
        if G < 1 or D % G:
            raise ValueError(f"filter groups {G} do not divide D={D}")
        H = D // G
        lo, hi = rows if rows is not None else (0, B * T)
        cu, ns = _cu(cu_seqlens)
        dx = np.empty((hi - lo, D))
        dw = np.empty((hi - lo, G, W))
        _check(self.lib.oracle_headwise_bwd(B, T, D, W, H, _ptr(x), _ptr(w), _ptr(dy), _ptr(cu), ns,
                                            int(bool(residual)), lo, hi, _ptr(dx), _ptr(dw)),
               "headwise_bwd")
        if rows is None:
            return dx.reshape(B, T, D), dw.reshape(B, T, G, W)
        return dx, dw

    def lowrank_fwd(self, x, z, U, W, *, cu_seqlens=None, residual=False, rows=None):
        """x (B,T,D), z (B,T,R), U (R, D*W) -> y."""
        x, z, U = _f64(x), _f64(z), _f64(U)
        B, T, D = x.shape
        R = z.shape[2]
        assert U.shape == (R, D * W)
        lo, hi = rows if rows is not None else (0, B * T)
        cu, ns = _cu(cu_seqlens)
        y = np.empty((hi - lo, D))
        _check(self.lib.oracle_lowrank_fwd(B, T, D, W, R, _ptr(x), _ptr(z), _ptr(U), _ptr(cu), ns,
                                           int(bool(residual)), lo, hi, _ptr(y)), "lowrank_fwd")
        return y.reshape(B, T, D) if rows is None else y

    def lowrank_bwd(self, x, z, U, dy, W, *, cu_seqlens=None, residual=False, rows=None,
                    channels=None):
        """-> (dx, dz, dU); dx/dz over token rows, dU (R, (d_hi-d_lo)*W) over channels."""
        x, z, U, dy = _f64(x), _f64(z), _f64(U), _f64(dy)
        B, T, D = x.shape
        R = z.shape[2]
        assert U.shape == (R, D * W)
        lo, hi = rows if rows is not None else (0, B * T)
        dlo, dhi = channels if channels is not None else (0, D)
        cu, ns = _cu(cu_seqlens)
        dx = np.empty((hi - lo, D))
        dz = np.empty((hi - lo, R))
        dU = np.empty((R, (dhi - dlo) * W))
        _check(self.lib.oracle_lowrank_bwd(B, T, D, W, R, _ptr(x), _ptr(z), _ptr(U), _ptr(dy),
                                           _ptr(cu), ns, int(bool(residual)), lo, hi, _ptr(dx),
                                           _ptr(dz), dlo, dhi, _ptr(dU)), "lowrank_bwd")
        if rows is None:
            return dx.reshape(B, T, D), dz.reshape(B, T, R), dU
        return dx, dz, dU

    def static_fwd(self, x, c, *, cu_seqlens=None, residual=False, rows=None):
        """x (B,T,D), c (D,W) one filter per channel -> y (B,T,D) (or compact rows)."""
        x, c = _f64(x), _f64(c)
        B, T, D = x.shape
        if c.ndim != 2 or c.shape[0] != D:
            raise ValueError(f"c must be (D, W) with D={D}, got {c.shape}")
        W = c.shape[1]
        lo, hi = rows if rows is not None else (0, B * T)
        cu, ns = _cu(cu_seqlens)
        y = np.empty((hi - lo, D))
        _check(self.lib.oracle_static_fwd(B, T, D, W, _ptr(x), _ptr(c), _ptr(cu), ns,
                                          int(bool(residual)), lo, hi, _ptr(y)), "static_fwd")
        return y.reshape(B, T, D) if rows is None else y

    def static_bwd(self, x, c, dy, *, cu_seqlens=None, residual=False, rows=None):
        """-> (dx, dc): dx over token rows, dc (D, W) summed over every token."""
        x, c, dy = _f64(x), _f64(c), _f64(dy)
        B, T, D = x.shape
        if c.ndim != 2 or c.shape[0] != D:
            raise ValueError(f"c must be (D, W) with D={D}, got {c.shape}")
        W = c.shape[1]
        lo, hi = rows if rows is not None else (0, B * T)
        cu, ns = _cu(cu_seqlens)
        dx = np.empty((hi - lo, D))
        dc = np.empty((D, W))
        _check(self.lib.oracle_static_bwd(B, T, D, W, _ptr(x), _ptr(c), _ptr(dy), _ptr(cu), ns,
                                          int(bool(residual)), lo, hi, _ptr(dx), _ptr(dc)), "static_bwd")
        return (dx.reshape(B, T, D) if rows is None else dx), dc

    def headwise_decode(self, x, w, state, *, residual=False):
        """One token per sequence: x (B,D), w (B,D/H,W), state (B,W-1,D) -> (y (B,D), new state)."""
        x, w = _f64(x), _f64(w)
        st = _f64(state).copy()
        B, D = x.shape
        G, W = w.shape[1], w.shape[2]
        if G < 1 or D % G or st.shape != (B, W - 1, D):
            raise ValueError("bad decode shapes")
        y = np.empty((B, D))
        _check(self.lib.oracle_headwise_decode(B, D, W, D // G, _ptr(x), _ptr(w), _ptr(st),
                                               int(bool(residual)), _ptr(y)), "headwise_decode")
        return y, st

    def lowrank_decode(self, x, z, U, state, W, *, residual=False):
        """x (B,D), z (B,R), U (R, D*W), state (B,W-1,D) -> (y (B,D), new state)."""
        x, z, U = _f64(x), _f64(z), _f64(U)
        st = _f64(state).copy()
        B, D = x.shape
        R = z.shape[1]
        if U.shape != (R, D * W) or st.shape != (B, W - 1, D):
            raise ValueError("bad decode shapes")
        y = np.empty((B, D))
        _check(self.lib.oracle_lowrank_decode(B, D, W, R, _ptr(x), _ptr(z), _ptr(U), _ptr(st),
                                              int(bool(residual)), _ptr(y)), "lowrank_decode")
        return y, st

    def state_from_prefill(self, x, W, *, cu_seqlens=None):
        """x (B,T,D) prefill inputs -> state (S, W-1, D) of every sequence's last W-1 tokens."""
        x = _f64(x)
        B, T, D = x.shape
        cu, ns = _cu(cu_seqlens)
        S = ns if cu is not None else B
        st = np.empty((S, W - 1, D))
        _check(self.lib.oracle_state_from_prefill(B, T, D, W, _ptr(x), _ptr(cu), ns, _ptr(st)),
               "state_from_prefill")
        return st

    # ------------------------------------------------------------------ RoPE
    # The rotation follows "RoFormer: Enhanced Transformer with Rotary Position
    # Embedding" (Su et al.), Section 3.4.2; the layer sits right before it on
    # the query and key projections (pages: Methodology, placement).

    def rope_table(self, max_pos, head_dim, base=10000.0):
        """-> (max_pos, head_dim/2, 2): cos and sin of m * base^(-2i/head_dim)."""
        t = np.empty((max_pos, head_dim // 2, 2))
        _check(self.lib.oracle_rope_table(max_pos, head_dim, float(base), _ptr(t)), "rope_table")
        return t

    def rope(self, v, *, rot, head_dim, base=10000.0, cu_seqlens=None, inverse=False, rows=None,
             shape=None):
        """Rotate channels [0, rot) of every row (pairs 2i, 2i+1 of each head of
        head_dim channels) by position-in-sequence times base^(-2i/head_dim).
        v is (B,T,D), or with rows=(lo, hi) and shape=(B, T) the compact rows
        (hi-lo, D).  inverse=True applies the transposed rotation."""
        v = _f64(v)
        if rows is None:
            B, T, D = v.shape
            lo, hi = 0, B * T
        else:
            (B, T), (lo, hi) = shape, rows
            D = v.shape[-1]
            if v.shape != (hi - lo, D):
                raise ValueError(f"rows {rows} do not match {v.shape}")
        cu, ns = _cu(cu_seqlens)
        out = np.empty_like(v)
        _check(self.lib.oracle_rope(B, T, D, int(rot), int(head_dim), float(base), _ptr(cu), ns,
                                    int(bool(inverse)), lo, hi, _ptr(v), _ptr(out)), "rope")
        return out

    def headwise_rope_fwd(self, x, w, *, rot, head_dim, base=10000.0, cu_seqlens=None,
                          residual=False, rows=None):
        """RoPE(rho*x + conv(x)): the head-wise layer, then the rotation of its
        first rot channels."""
        y = self.headwise_fwd(x, w, cu_seqlens=cu_seqlens, residual=residual, rows=rows)
        B, T, _ = np.shape(x)
        return self.rope(y, rot=rot, head_dim=head_dim, base=base, cu_seqlens=cu_seqlens, rows=rows,
                         shape=(B, T))

    def rope_at(self, v, positions, *, rot, head_dim, base=10000.0):
        """v (B, D): row b, the newest token of sequence b, rotated at position positions[b]."""
        v = _f64(v)
        pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
        B, D = v.shape
        if pos.shape != (B,):
            raise ValueError("one position per row")
        out = np.empty_like(v)
        _check(self.lib.oracle_rope_at(B, D, int(rot), int(head_dim), float(base), _ptr(pos), _ptr(v),
                                       _ptr(out)), "rope_at")
        return out

    def headwise_rope_decode(self, x, w, state, positions, *, rot, head_dim, base=10000.0, residual=False):
        """One decoding step of the head-wise layer, then the rotation of its
        output at each sequence's position -> (y (B, D), new state)."""
        y, st = self.headwise_decode(x, w, state, residual=residual)
        return self.rope_at(y, positions, rot=rot, head_dim=head_dim, base=base), st

    def headwise_rope_bwd(self, x, w, dy, *, rot, head_dim, base=10000.0, cu_seqlens=None,
                          residual=False, rows=None):
        """-> (dx, dw).  The rotation is orthogonal and comes last, so the
        layer's output gradient is the transposed rotation of dy."""
        ds = self.rope(dy, rot=rot, head_dim=head_dim, base=base, cu_seqlens=cu_seqlens, inverse=True)
        return self.headwise_bwd(x, w, ds, cu_seqlens=cu_seqlens, residual=residual, rows=rows)

    def generate(self, h, V, *, rows=None):
        """w = h V^T: h (N, K) hidden states, V (C, K) the generator's weight ->
        (rows, C) for token rows [lo, hi) (default all)."""
        h, V = _f64(h), _f64(V)
        h = h.reshape(-1, h.shape[-1])
        N, K = h.shape
        C = V.shape[0]
        if V.shape != (C, K):
            raise ValueError(f"V must be (C, {K}), got {V.shape}")
        lo, hi = rows if rows is not None else (0, N)
        w = np.empty((hi - lo, C))
        _check(self.lib.oracle_generate(N, K, C, _ptr(h), _ptr(V), lo, hi, _ptr(w)), "generate")
        return w

    def headwise_gen_fwd(self, h, V, x, *, W, cu_seqlens=None, residual=False, rows=None):
        """The head-wise layer whose filters come from the hidden state:
        w[n, g, k] = sum_j h[n, j] V[g*W + k, j] (Methodology, parametrization:
        a learned linear map of the current hidden state), then y as
        headwise_fwd.  h (B,T,K), V (G*W, K), x (B,T,D) -> y (or compact rows)."""
        x = _f64(x)
        B, T, D = x.shape
        N = B * T
        G = _f64(V).shape[0] // W
        lo, hi = rows if rows is not None else (0, N)
        w = np.zeros((N, G * W))
        w[lo:hi] = self.generate(h, V, rows=(lo, hi))  # y of row n reads w of row n only
        return self.headwise_fwd(x, w.reshape(B, T, G, W), cu_seqlens=cu_seqlens, residual=residual, rows=rows)

    def headwise_gen_bwd(self, h, V, x, dy, *, W, cu_seqlens=None, residual=False, rows=None, groups=None):
        """-> (dx, dh, dV) for L = <dy, y>: dx, dh over token rows [lo, hi)
        (default all), dV (rows g*W + k for groups [g_lo, g_hi), K) summed
        over every token (default all groups).  dw is the head-wise layer's
        filter gradient; dh = dw V and dV = dw^T h are the chain rule of the
        linear map."""
        h, V, x, dy = _f64(h), _f64(V), _f64(x), _f64(dy)
        B, T, D = x.shape
        N = B * T
        K = h.shape[-1]
        C = V.shape[0]
        G = C // W
        H = D // G
        lo, hi = rows if rows is not None else (0, N)
        glo, ghi = groups if groups is not None else (0, G)
        # dx of rows [lo, hi) reads the filters of rows up to hi + W - 2
        w = np.zeros((N, C))
        whi = min(N, hi + W - 1)
        if hi > lo:
            w[lo:whi] = self.generate(h, V, rows=(lo, whi))
        dx, dw = self.headwise_bwd(x, w.reshape(B, T, G, W), dy, cu_seqlens=cu_seqlens, residual=residual,
                                   rows=(lo, hi))
        dh = np.empty((hi - lo, K))
        _check(self.lib.oracle_generate_bwd_h(K, C, _ptr(np.ascontiguousarray(dw.reshape(hi - lo, C))), _ptr(V),
                                              hi - lo, _ptr(dh)), "generate_bwd_h")
        # dV of groups [glo, ghi): the filter gradient of those groups' channels
        # over every token (it does not depend on w)
        dV = np.empty(((ghi - glo) * W, K))
        if ghi > glo:
            xs = np.ascontiguousarray(x[..., glo * H:ghi * H])
            gs = np.ascontiguousarray(dy[..., glo * H:ghi * H])
            _, dws = self.headwise_bwd(xs, np.zeros((B, T, ghi - glo, W)), gs, cu_seqlens=cu_seqlens)
            dws = np.ascontiguousarray(dws.reshape(N, (ghi - glo) * W))
            _check(self.lib.oracle_generate_bwd_v(N, K, (ghi - glo) * W, _ptr(dws), _ptr(h.reshape(N, K)), 0,
                                                  (ghi - glo) * W, _ptr(dV)), "generate_bwd_v")
        if rows is None:
            return dx.reshape(B, T, D), dh.reshape(B, T, K), dV
        return dx, dh, dV

    def lowrank_rope_fwd(self, x, z, U, W, *, rot, head_dim, base=10000.0, cu_seqlens=None,
                         residual=False, rows=None):
        """RoPE(rho*x + conv(x)) with the low-rank filters z U: the low-rank
        layer on the query, key and value projections (ES summary,
        Metodología: placement right before the rotary embedding), then the
        rotation of its first rot channels."""
        y = self.lowrank_fwd(x, z, U, W, cu_seqlens=cu_seqlens, residual=residual, rows=rows)
        B, T, _ = np.shape(x)
        return self.rope(y, rot=rot, head_dim=head_dim, base=base, cu_seqlens=cu_seqlens, rows=rows,
                         shape=(B, T))

    def lowrank_rope_bwd(self, x, z, U, dy, W, *, rot, head_dim, base=10000.0, cu_seqlens=None,
                         residual=False, rows=None, channels=None):
        """-> (dx, dz, dU): the low-rank layer's backward on the transposed
        rotation of dy (the rotation is orthogonal and comes last)."""
        ds = self.rope(dy, rot=rot, head_dim=head_dim, base=base, cu_seqlens=cu_seqlens, inverse=True)
        return self.lowrank_bwd(x, z, U, ds, W, cu_seqlens=cu_seqlens, residual=residual, rows=rows,
                                channels=channels)


def num_threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(load().oracle_num_threads())


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def headwise_fwd(*a, **k):
    return default().headwise_fwd(*a, **k)


def headwise_bwd(*a, **k):
    return default().headwise_bwd(*a, **k)


def lowrank_fwd(*a, **k):
    return default().lowrank_fwd(*a, **k)


def lowrank_bwd(*a, **k):
    return default().lowrank_bwd(*a, **k)


def static_fwd(*a, **k):
    return default().static_fwd(*a, **k)


def static_bwd(*a, **k):
    return default().static_bwd(*a, **k)


def headwise_decode(*a, **k):
    return default().headwise_decode(*a, **k)


def lowrank_decode(*a, **k):
    return default().lowrank_decode(*a, **k)


def state_from_prefill(*a, **k):
    return default().state_from_prefill(*a, **k)


def rope_table(*a, **k):
    return default().rope_table(*a, **k)


def rope(*a, **k):
    return default().rope(*a, **k)


def headwise_rope_fwd(*a, **k):
    return default().headwise_rope_fwd(*a, **k)


def generate(*a, **k):
    return default().generate(*a, **k)


def headwise_gen_fwd(*a, **k):
    return default().headwise_gen_fwd(*a, **k)


def headwise_gen_bwd(*a, **k):
    return default().headwise_gen_bwd(*a, **k)


def lowrank_rope_fwd(*a, **k):
    return default().lowrank_rope_fwd(*a, **k)


def lowrank_rope_bwd(*a, **k):
    return default().lowrank_rope_bwd(*a, **k)


def headwise_rope_bwd(*a, **k):
    return default().headwise_rope_bwd(*a, **k)


def rope_at(*a, **k):
    return default().rope_at(*a, **k)


def headwise_rope_decode(*a, **k):
    return default().headwise_rope_decode(*a, **k)
