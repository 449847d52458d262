"""Thin Python binding of libdsc.so (include/dsc.h).

Argument marshalling only: shapes, dtype codes, device pointers and the
current HIP stream are read from torch tensors and passed through ctypes;
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if libdsc.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsc.so")

DSC_FP32, DSC_BF16 = 0, 1
STATUS = {0: "DSC_SUCCESS", 1: "DSC_ERR_NULL", 2: "DSC_ERR_SHAPE", 3: "DSC_ERR_UNSUPPORTED",
          4: "DSC_ERR_ALIGNMENT", 5: "DSC_ERR_ALIAS", 6: "DSC_ERR_WORKSPACE", 7: "DSC_ERR_HIP"}

_lib = None


class DscError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m input_dependent_short_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, p, i = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
        L.dsc_headwise_fwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, i32, i32, p]
        L.dsc_headwise_bwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, p, i32, i32, p, p]
        L.dsc_lowrank_fwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, p, i32, i32, p]
        L.dsc_lowrank_bwd_workspace_size.argtypes = [i, i64, i64, i64, i32, i32]
        L.dsc_lowrank_bwd_workspace_size.restype = ctypes.c_size_t
        L.dsc_lowrank_bwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, p, p, i32, i32, p, p, p,
                                      p, ctypes.c_size_t]
        L.dsc_lowrank_bwd_deterministic_workspace_size.argtypes = [i, i64, i64, i64, i32, i32]
        L.dsc_lowrank_bwd_deterministic_workspace_size.restype = ctypes.c_size_t
        L.dsc_lowrank_bwd_deterministic.argtypes = L.dsc_lowrank_bwd.argtypes
        L.dsc_lowrank_bwd_noalloc.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, p, p, i32, i32, p, p, p]
        L.dsc_static_fwd.argtypes = [p, i, i64, i64, i64, i32, p, p, p, i32, i32, p]
        L.dsc_static_bwd.argtypes = [p, i, i64, i64, i64, i32, p, p, p, p, i32, i32, p, p]
        L.dsc_static_bwd_deterministic_workspace_size.argtypes = [i, i64, i64, i64, i32]
        L.dsc_static_bwd_deterministic_workspace_size.restype = ctypes.c_size_t
        L.dsc_static_bwd_deterministic.argtypes = [p, i, i64, i64, i64, i32, p, p, p, p, i32, i32, p, p, p,
                                                   ctypes.c_size_t]
        L.dsc_headwise_decode.argtypes = [p, i, i64, i64, i32, i32, p, p, p, i32, p]
        L.dsc_lowrank_decode.argtypes = [p, i, i64, i64, i32, i32, p, p, p, p, i32, p]
        L.dsc_state_from_prefill.argtypes = [p, i, i64, i64, i64, i32, p, p, i32, p]
        L.dsc_rope_table.argtypes = [p, i64, i32, ctypes.c_double, p]
        L.dsc_headwise_rope_decode.argtypes = [p, i, i64, i64, i32, i32, p, p, p, i32, i64, i32, p, i64, p, p]
        L.dsc_headwise_rope_fwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, i32, i32, i64, i32, p, i64, p]
        L.dsc_headwise_rope_bwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, p, i32, i32, i64, i32, p, i64,
                                            p, p]
        L.dsc_lowrank_rope_fwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, p, i32, i32, i64, i32, p, i64, p]
        L.dsc_lowrank_rope_bwd.argtypes = [p, i, i64, i64, i64, i32, i32, p, p, p, p, p, i32, i32, i64, i32, p, i64,
                                           p, p, p, p, ctypes.c_size_t]
        L.dsc_headwise_gen_fwd.argtypes = [p, i, i64, i64, i64, i32, i32, i64, p, p, p, p, i32, i32, p]
        L.dsc_headwise_gen_bwd_workspace_size.argtypes = [i, i64, i64, i64, i32, i32, i64]
        L.dsc_headwise_gen_bwd_workspace_size.restype = ctypes.c_size_t
        L.dsc_headwise_gen_bwd.argtypes = [p, i, i64, i64, i64, i32, i32, i64, p, p, p, p, p, i32, i32, p, p, p,
                                           p, ctypes.c_size_t]
        L.dsc_generate_filters.argtypes = [p, i, i64, i64, i64, p, p, p]
        L.dsc_bench_stream.argtypes = [p, p, i64, p, i64, i32, i32, i32, i32, i64]
        for f in ("dsc_bench_stream", "dsc_lowrank_bwd_noalloc", "dsc_headwise_fwd", "dsc_headwise_bwd", "dsc_lowrank_fwd", "dsc_lowrank_bwd",
                  "dsc_lowrank_bwd_deterministic", "dsc_static_bwd_deterministic",
                  "dsc_static_fwd", "dsc_static_bwd", "dsc_headwise_decode", "dsc_lowrank_decode",
                  "dsc_state_from_prefill", "dsc_rope_table", "dsc_headwise_rope_fwd",
                  "dsc_headwise_rope_bwd", "dsc_headwise_rope_decode", "dsc_lowrank_rope_fwd",
                  "dsc_lowrank_rope_bwd", "dsc_headwise_gen_fwd", "dsc_headwise_gen_bwd", "dsc_generate_filters",
                  "dsc_abi_version"):
            getattr(L, f).restype = ctypes.c_int
        L.dsc_status_string.argtypes = [i]
        L.dsc_status_string.restype = ctypes.c_char_p
        L.dsc_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSC_FP32
    if t.dtype == torch.bfloat16:
        return DSC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _seq(cu_seqlens: torch.Tensor | None):
    if cu_seqlens is None:
        return None, 0
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    return _ptr(cu_seqlens), cu_seqlens.numel() - 1


def _check(rc: int) -> None:
    if rc != 0:
        raise DscError(rc, lib().dsc_last_error().decode())


def dsc_headwise_fwd(x, w, y, *, cu_seqlens=None, residual=False, stream=None) -> None:
    """y = rho*x + dynamic conv of x with head-wise filters w (B,T,D/H,W)."""
    B, T, D = x.shape
    G, W = w.shape[2], w.shape[3]
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_headwise_fwd(_stream(stream), _dtype_code(x), B, T, D, W, D // G if G else 0,
                                  _ptr(x), _ptr(w), cu, ns, int(bool(residual)), _ptr(y)))


def dsc_headwise_bwd(x, w, dy, dx, dw, *, cu_seqlens=None, residual=False, stream=None) -> None:
    B, T, D = x.shape
    G, W = w.shape[2], w.shape[3]
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_headwise_bwd(_stream(stream), _dtype_code(x), B, T, D, W, D // G if G else 0,
                                  _ptr(x), _ptr(w), _ptr(dy), cu, ns, int(bool(residual)),
                                  _ptr(dx), _ptr(dw)))


def dsc_rope_table(table, *, base=10000.0, stream=None) -> None:
    """Fill table (max_pos, head_dim/2, 2) fp32 with cos, sin of m * base^(-2i/head_dim)."""
    if table.dtype != torch.float32 or table.dim() != 3 or table.shape[2] != 2:
        raise ValueError("table must be fp32 (max_pos, head_dim/2, 2)")
    _check(lib().dsc_rope_table(_stream(stream), table.shape[0], 2 * table.shape[1], float(base), _ptr(table)))


def _table(table, head_dim):
    if table is None:
        return None, 0
    if table.dtype != torch.float32 or table.dim() != 3 or table.shape[1:] != (head_dim // 2, 2):
        raise ValueError(f"table must be fp32 (max_pos, {head_dim // 2}, 2)")
    return _ptr(table), table.shape[0]


def dsc_headwise_rope_fwd(x, w, y, *, rot, head_dim, table, cu_seqlens=None, residual=False,
                          stream=None) -> None:
    """y = rotary embedding (channels [0, rot), heads of head_dim) of the head-wise layer's output."""
    B, T, D = x.shape
    G, W = w.shape[2], w.shape[3]
    cu, ns = _seq(cu_seqlens)
    tp, max_pos = _table(table, head_dim)
    _check(lib().dsc_headwise_rope_fwd(_stream(stream), _dtype_code(x), B, T, D, W, D // G if G else 0,
                                       _ptr(x), _ptr(w), cu, ns, int(bool(residual)), int(rot), int(head_dim),
                                       tp, max_pos, _ptr(y)))


def dsc_headwise_rope_bwd(x, w, dy, dx, dw, *, rot, head_dim, table, cu_seqlens=None, residual=False,
                          stream=None) -> None:
    B, T, D = x.shape
    G, W = w.shape[2], w.shape[3]
    cu, ns = _seq(cu_seqlens)
    tp, max_pos = _table(table, head_dim)
    _check(lib().dsc_headwise_rope_bwd(_stream(stream), _dtype_code(x), B, T, D, W, D // G if G else 0,
                                       _ptr(x), _ptr(w), _ptr(dy), cu, ns, int(bool(residual)), int(rot),
                                       int(head_dim), tp, max_pos, _ptr(dx), _ptr(dw)))


def dsc_headwise_rope_decode(x, w, state, y, positions, *, rot, head_dim, table, residual=False,
                             stream=None) -> None:
    """One decoding step (x (B,D), w (B,D/H,W), state (B,W-1,D) updated in place),
    y rotated at positions (B,) int32 on the device."""
    B, D = x.shape
    G, W = w.shape[1], w.shape[2]
    if positions.dtype != torch.int32:
        raise TypeError("positions must be int32")
    tp, max_pos = _table(table, head_dim)
    _check(lib().dsc_headwise_rope_decode(_stream(stream), _dtype_code(x), B, D, W, D // G if G else 0, _ptr(x),
                                          _ptr(w), _ptr(state), int(bool(residual)), int(rot), int(head_dim), tp,
                                          max_pos, _ptr(positions), _ptr(y)))


def dsc_headwise_gen_fwd(h, V, x, y, *, W, cu_seqlens=None, residual=False, stream=None) -> None:
    """y = head-wise layer on x with filters w = h V^T generated on chip (V is (G*W, K))."""
    B, T, D = x.shape
    K = h.shape[2]
    G = V.shape[0] // W if W else 0
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_headwise_gen_fwd(_stream(stream), _dtype_code(x), B, T, D, W, D // G if G else 0, K,
                                      _ptr(h), _ptr(V), _ptr(x), cu, ns, int(bool(residual)), _ptr(y)))


def dsc_generate_filters(h, V, w, stream=None) -> None:
    """w (N, C) = h (N, K) V (C, K)^T on the matrix cores (bf16)."""
    K = h.shape[-1]
    N = h.numel() // K if K else 0
    C = V.shape[0]
    _check(lib().dsc_generate_filters(_stream(stream), _dtype_code(h), N, K, C, _ptr(h), _ptr(V), _ptr(w)))


def dsc_headwise_gen_bwd_workspace_size(dtype: torch.dtype, B: int, T: int, D: int, W: int, H: int, K: int) -> int:
    code = DSC_BF16 if dtype == torch.bfloat16 else DSC_FP32
    return int(lib().dsc_headwise_gen_bwd_workspace_size(code, B, T, D, W, H, K))


def dsc_headwise_gen_bwd(h, V, x, dy, dx, dh, dV, workspace=None, *, W, cu_seqlens=None, residual=False,
                         stream=None) -> None:
    B, T, D = x.shape
    K = h.shape[2]
    G = V.shape[0] // W if W else 0
    cu, ns = _seq(cu_seqlens)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsc_headwise_gen_bwd(_stream(stream), _dtype_code(x), B, T, D, W, D // G if G else 0, K,
                                      _ptr(h), _ptr(V), _ptr(x), _ptr(dy), cu, ns, int(bool(residual)), _ptr(dx),
                                      _ptr(dh), _ptr(dV), _ptr(workspace), ws_bytes))


def dsc_lowrank_fwd(x, z, U, y, *, W, cu_seqlens=None, residual=False, stream=None) -> None:
    """y = rho*x + dynamic conv of x with filters z U (U is (R, D*W))."""
    B, T, D = x.shape
    R = z.shape[2]
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_lowrank_fwd(_stream(stream), _dtype_code(x), B, T, D, W, R, _ptr(x), _ptr(z),
                                 _ptr(U), cu, ns, int(bool(residual)), _ptr(y)))


def dsc_lowrank_rope_fwd(x, z, U, y, *, W, rot, head_dim, table, cu_seqlens=None, residual=False,
                         stream=None) -> None:
    """y = rotary embedding (channels [0, rot), heads of head_dim) of the low-rank layer's output."""
    B, T, D = x.shape
    R = z.shape[2]
    cu, ns = _seq(cu_seqlens)
    tp, max_pos = _table(table, head_dim)
    _check(lib().dsc_lowrank_rope_fwd(_stream(stream), _dtype_code(x), B, T, D, W, R, _ptr(x), _ptr(z),
                                      _ptr(U), cu, ns, int(bool(residual)), int(rot), int(head_dim), tp, max_pos,
                                      _ptr(y)))


def dsc_lowrank_rope_bwd(x, z, U, dy, dx, dz, dU, workspace=None, *, W, rot, head_dim, table, cu_seqlens=None,
                         residual=False, stream=None) -> None:
    B, T, D = x.shape
    R = z.shape[2]
    cu, ns = _seq(cu_seqlens)
    tp, max_pos = _table(table, head_dim)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsc_lowrank_rope_bwd(_stream(stream), _dtype_code(x), B, T, D, W, R, _ptr(x), _ptr(z),
                                      _ptr(U), _ptr(dy), cu, ns, int(bool(residual)), int(rot), int(head_dim), tp,
                                      max_pos, _ptr(dx), _ptr(dz), _ptr(dU), _ptr(workspace), ws_bytes))


def dsc_lowrank_bwd_workspace_size(dtype: torch.dtype, B: int, T: int, D: int, W: int, R: int) -> int:
    code = DSC_BF16 if dtype == torch.bfloat16 else DSC_FP32
    return int(lib().dsc_lowrank_bwd_workspace_size(code, B, T, D, W, R))


def dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, workspace=None, *, W, cu_seqlens=None,
                    residual=False, stream=None) -> None:
    B, T, D = x.shape
    R = z.shape[2]
    cu, ns = _seq(cu_seqlens)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsc_lowrank_bwd(_stream(stream), _dtype_code(x), B, T, D, W, R, _ptr(x), _ptr(z),
                                 _ptr(U), _ptr(dy), cu, ns, int(bool(residual)), _ptr(dx), _ptr(dz),
                                 _ptr(dU), _ptr(workspace), ws_bytes))


def dsc_lowrank_bwd_noalloc(x, z, U, dy, dx, dz, dU, *, W, cu_seqlens=None, residual=False,
                            stream=None) -> None:
    """dsc_lowrank_bwd without a workspace (the library's built-in device scratch; B*T*R <= 4,194,304)."""
    B, T, D = x.shape
    R = z.shape[2]
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_lowrank_bwd_noalloc(_stream(stream), _dtype_code(x), B, T, D, W, R, _ptr(x), _ptr(z),
                                         _ptr(U), _ptr(dy), cu, ns, int(bool(residual)), _ptr(dx), _ptr(dz),
                                         _ptr(dU)))


def dsc_lowrank_bwd_deterministic_workspace_size(dtype: torch.dtype, B: int, T: int, D: int, W: int,
                                                 R: int) -> int:
    code = DSC_BF16 if dtype == torch.bfloat16 else DSC_FP32
    return int(lib().dsc_lowrank_bwd_deterministic_workspace_size(code, B, T, D, W, R))


def dsc_lowrank_bwd_deterministic(x, z, U, dy, dx, dz, dU, workspace=None, *, W, cu_seqlens=None,
                                  residual=False, stream=None) -> None:
    """dsc_lowrank_bwd with dz and dU summed in a fixed order (bitwise reproducible)."""
    B, T, D = x.shape
    R = z.shape[2]
    cu, ns = _seq(cu_seqlens)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsc_lowrank_bwd_deterministic(_stream(stream), _dtype_code(x), B, T, D, W, R, _ptr(x), _ptr(z),
                                               _ptr(U), _ptr(dy), cu, ns, int(bool(residual)), _ptr(dx),
                                               _ptr(dz), _ptr(dU), _ptr(workspace), ws_bytes))


def dsc_static_fwd(x, c, y, *, cu_seqlens=None, residual=False, stream=None) -> None:
    """y = rho*x + static causal conv of x with one filter per channel, c (D, W)."""
    B, T, D = x.shape
    W = c.shape[1]
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_static_fwd(_stream(stream), _dtype_code(x), B, T, D, W, _ptr(x), _ptr(c), cu, ns,
                                int(bool(residual)), _ptr(y)))


def dsc_static_bwd(x, c, dy, dx, dc, *, cu_seqlens=None, residual=False, stream=None) -> None:
    """dx (B,T,D) and dc (D, W) fp32 of the static conv."""
    B, T, D = x.shape
    W = c.shape[1]
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_static_bwd(_stream(stream), _dtype_code(x), B, T, D, W, _ptr(x), _ptr(c), _ptr(dy),
                                cu, ns, int(bool(residual)), _ptr(dx), _ptr(dc)))


def dsc_static_bwd_deterministic_workspace_size(dtype: torch.dtype, B: int, T: int, D: int, W: int) -> int:
    code = DSC_BF16 if dtype == torch.bfloat16 else DSC_FP32
    return int(lib().dsc_static_bwd_deterministic_workspace_size(code, B, T, D, W))


def dsc_static_bwd_deterministic(x, c, dy, dx, dc, workspace=None, *, cu_seqlens=None, residual=False,
                                 stream=None) -> None:
    """dsc_static_bwd with dc summed in a fixed order (bitwise reproducible)."""
    B, T, D = x.shape
    W = c.shape[1]
    cu, ns = _seq(cu_seqlens)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsc_static_bwd_deterministic(_stream(stream), _dtype_code(x), B, T, D, W, _ptr(x), _ptr(c),
                                              _ptr(dy), cu, ns, int(bool(residual)), _ptr(dx), _ptr(dc),
                                              _ptr(workspace), ws_bytes))


def dsc_headwise_decode(x, w, state, y, *, residual=False, stream=None) -> None:
    """One token per sequence: x (B,D), w (B,D/H,W), state (B,W-1,D) updated in place, y (B,D)."""
    B, D = x.shape
    G, W = w.shape[1], w.shape[2]
    _check(lib().dsc_headwise_decode(_stream(stream), _dtype_code(x), B, D, W, D // G if G else 0, _ptr(x),
                                     _ptr(w), _ptr(state), int(bool(residual)), _ptr(y)))


def dsc_lowrank_decode(x, z, U, state, y, *, W, residual=False, stream=None) -> None:
    """One token per sequence: x (B,D), z (B,R), U (R, D*W), state (B,W-1,D) updated in place."""
    B, D = x.shape
    R = z.shape[1]
    _check(lib().dsc_lowrank_decode(_stream(stream), _dtype_code(x), B, D, W, R, _ptr(x), _ptr(z), _ptr(U),
                                    _ptr(state), int(bool(residual)), _ptr(y)))


def dsc_state_from_prefill(x, state, *, W, cu_seqlens=None, stream=None) -> None:
    """state (S, W-1, D) <- the last W-1 inputs of every sequence of x (B,T,D)."""
    B, T, D = x.shape
    cu, ns = _seq(cu_seqlens)
    _check(lib().dsc_state_from_prefill(_stream(stream), _dtype_code(x), B, T, D, W, _ptr(x), cu, ns,
                                        _ptr(state)))


def dsc_bench_stream(src, read_bytes: int, dst, write_bytes: int, *, unroll=4, load_nt=False, store_nt=False,
                     chunked=False, blocks=0, stream=None) -> None:
    """Streaming measurement kernel (include/dsc_bench.h): reads read_bytes of
    src and writes write_bytes of dst (raw device buffers, any dtype)."""
    _check(lib().dsc_bench_stream(_stream(stream), _ptr(src), int(read_bytes), _ptr(dst), int(write_bytes),
                                  int(unroll), int(bool(load_nt)), int(bool(store_nt)), int(bool(chunked)),
                                  int(blocks)))


def dsc_abi_version() -> int:
    return int(lib().dsc_abi_version())
