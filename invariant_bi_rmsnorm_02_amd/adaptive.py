"""Python binding of libbi_adaptive.so (include/bi_adaptive.h): the
shape-adaptive comparators used to measure the cost of batch invariance.

They are NOT batch-invariant (a split count follows the shape of the batch);
tests use them as a negative control and bench.py times them beside libbi.so.
Argument marshalling only, as in the package's main binding.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import BiError, _dev, _rows, _stream, _tokens, _cache_geom, status_str  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbi_adaptive.so")

_i32, _i64, _f32, _sz, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_SIGNATURES = {
    "bia_gemm_splits": (_i32, [_i64, _i64, _i64]),
    "bia_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bia_gemm": (_i32, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _sz, _p]),
    "bia_attn_decode_split_keys": (_i32, [_i32, _i32, _i32, _i32]),
    "bia_attn_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "bia_attn_decode": (_i32, [_p, _i64, _p, _p, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                               _p, _p, _p, _sz, _p]),
    "bia_rmsnorm_slices": (_i32, [_i64, _i64]),
    "bia_rmsnorm_workspace_bytes": (_sz, [_i64, _i64]),
    "bia_rmsnorm": (_i32, [_p, _i64, _p, _f32, _p, _i64, _i64, _i64, _p, _sz, _p]),
}
_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise BiError(fn, status)


def _ws(need: int, workspace: Optional[torch.Tensor], device) -> torch.Tensor:
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace


def gemm_splits(m: int, n: int, k: int) -> int:
    return int(lib().bia_gemm_splits(m, n, k))


def bia_gemm(a: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    m, k = a.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _dev(out, "out", torch.bfloat16)
    ws = _ws(int(lib().bia_gemm_workspace_bytes(m, n, k)), workspace, a.device)
    _check("bia_gemm", lib().bia_gemm(a.data_ptr(), _rows(a, "a"), w.data_ptr(), _rows(w, "w"), out.data_ptr(),
                                      _rows(out, "out"), m, n, k, ws.data_ptr(), ws.numel() * ws.element_size(),
                                      _stream(stream)))
    return out


def decode_split_keys(num_seqs: int, num_kv_heads: int, max_seq_len: int, page_size: int) -> int:
    """Keys per split the comparator picks for this batch (256: libbi's own decode)."""
    return int(lib().bia_attn_decode_split_keys(num_seqs, num_kv_heads, max_seq_len, page_size))


def bia_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    pages, hkv, ps, d = _cache_geom(k_cache, v_cache)
    _dev(q, "q", torch.bfloat16)
    b, hq, _ = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    ws = _ws(int(lib().bia_attn_decode_workspace_bytes(b, hq, hkv, d, int(max_seq_len), ps)), workspace, q.device)
    _check("bia_attn_decode", lib().bia_attn_decode(
        q.data_ptr(), _tokens(q, "q"), k_cache.data_ptr(), v_cache.data_ptr(), pages, block_table.data_ptr(),
        block_table.shape[1], seq_lens.data_ptr(), b, int(max_seq_len), hq, hkv, d, ps, float(softmax_scale),
        out.data_ptr(), lse.data_ptr() if lse is not None else None, ws.data_ptr(),
        ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


def rmsnorm_slices(rows: int, hidden: int) -> int:
    return int(lib().bia_rmsnorm_slices(rows, hidden))


def bia_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(x, "x", torch.bfloat16)
    _dev(gamma, "gamma", torch.bfloat16)
    rows, hidden = x.shape
    if out is None:
        out = torch.empty_like(x)
    ws = _ws(int(lib().bia_rmsnorm_workspace_bytes(rows, hidden)), workspace, x.device)
    _check("bia_rmsnorm", lib().bia_rmsnorm(x.data_ptr(), _rows(x, "x"), gamma.data_ptr(), float(eps), out.data_ptr(),
                                            _rows(out, "out"), rows, hidden, ws.data_ptr(),
                                            ws.numel() * ws.element_size(), _stream(stream)))
    return out
