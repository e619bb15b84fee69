"""Python binding of libbi.so (include/bi.h): argument marshalling only.

Every operation runs in the HIP library.  PyTorch supplies device memory and
the current HIP stream; the wrappers check devices, dtypes and shapes (so a
host pointer can never reach a kernel), pass ``data_ptr()`` values and sizes to
the C entry points of the same name, and raise ``BiError`` on a negative
status.  There is no fallback: if libbi.so is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbi.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "bi.h")

BI_OK, BI_ERR_INVALID_ARG, BI_ERR_UNSUPPORTED, BI_ERR_WORKSPACE, BI_ERR_HIP = 0, -1, -2, -3, -4
BI_BF16, BI_F32 = 0, 1
BI_KV_CHUNK = 256
BI_DECODE_SCRATCH_BYTES = 128 << 20

_c_i32, _c_i64, _c_f32, _c_size, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "bi_status_str": (ctypes.c_char_p, [_c_i32]),
    "bi_version": (ctypes.c_char_p, []),
    "bi_rmsnorm": (_c_i32, [_c_p, _c_i64, _c_p, _c_f32, _c_p, _c_i64, _c_i64, _c_i64, _c_p]),
    "bi_gemm": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_i32, _c_i64, _c_i64, _c_i64, _c_p]),
    "bi_gemm_tile": (_c_i32, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p]),
    "bi_gemm_add": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p]),
    "bi_gemm_silu_mul": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p]),
    "bi_kv_append": (_c_i32, [_c_p, _c_p, _c_i64, _c_p, _c_i32, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p]),
    "bi_attn_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "bi_attn_decode": (_c_i32, [_c_p, _c_i64, _c_p, _c_p, _c_i32, _c_p, _c_i32, _c_p, _c_i32, _c_i32, _c_i32,
                                _c_i32, _c_i32, _c_i32, _c_f32, _c_p, _c_p, _c_p, _c_size, _c_p]),
    "bi_attn_decode_noalloc": (_c_i32, [_c_p, _c_i64, _c_p, _c_p, _c_i32, _c_p, _c_i32, _c_p, _c_i32, _c_i32,
                                        _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_p, _c_p, _c_p]),
    "bi_attn_prefill_workspace_bytes": (_c_size, [_c_i32]),
    "bi_attn_prefill": (_c_i32, [_c_p, _c_i64, _c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_i32,
                                 _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_p, _c_p, _c_p, _c_size, _c_p]),
    "bi_log_softmax": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_p]),
    "bi_moe_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "bi_moe_route": (_c_i32, [_c_p, _c_i64, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p]),
    "bi_moe_ffn": (_c_i32, [_c_p, _c_i64, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_i32,
                            _c_p, _c_i64, _c_p, _c_size, _c_p]),
    "bi_lm_head_logprobs_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "bi_lm_head_logprobs": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64,
                                     _c_p, _c_size, _c_p]),
    "bi_lm_head_greedy_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "bi_lm_head_greedy": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_size,
                                   _c_p]),
    "bi_add": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_p]),
    "bi_silu_mul": (_c_i32, [_c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_p]),
}

_lib: Optional[ctypes.CDLL] = None


class BiError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")
        self.status = status


def header_symbols() -> list:
    """Names of the functions include/bi.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|bi_status|size_t)\s+(bi_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """Load libbi.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(or python invariant_bi_rmsnorm_02_amd/_build.py)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_str(status: int) -> str:
    return lib().bi_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != BI_OK:
        raise BiError(fn, status)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _tokens(t: torch.Tensor, name: str) -> int:
    """Token stride (elements) of a [T, H, D] tensor whose heads and dims are contiguous."""
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1) or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{name} must be [T, heads, dim] with heads and dims contiguous")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1] * t.shape[2], t.stride(0))


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


# ---------------------------------------------------------------- entry points

def bi_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    _dev(x, "x", torch.bfloat16)
    _dev(gamma, "gamma", torch.bfloat16)
    rows, hidden = x.shape
    if gamma.shape != (hidden,) or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous [hidden] tensor")
    if out is None:
        out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != x.shape:
        raise ValueError("out shape")
    _check("bi_rmsnorm", lib().bi_rmsnorm(x.data_ptr(), _rows(x, "x"), gamma.data_ptr(), float(eps),
                                          out.data_ptr(), _rows(out, "out"), rows, hidden, _stream(stream)))
    return out


def bi_gemm(a: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
            out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """out[m, n] = sum_k a[m, k] * w[n, k]."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    m, k = a.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    if out.dtype not in (torch.bfloat16, torch.float32) or not out.is_cuda or out.shape != (m, n):
        raise ValueError("out must be a GPU [m, n] bf16 or fp32 tensor")
    cdt = BI_F32 if out.dtype == torch.float32 else BI_BF16
    _check("bi_gemm", lib().bi_gemm(a.data_ptr(), _rows(a, "a"), w.data_ptr(), _rows(w, "w"), out.data_ptr(),
                                    _rows(out, "out"), cdt, m, n, k, _stream(stream)))
    return out


class _GemmConfig(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in ("tile_n", "tile_m", "waves_n", "waves_m", "stages", "stage_k", "per_cu",
                                              "stream_w")]


def gemm_config(m: int, n: int, k: int, lda: Optional[int] = None, ldw: Optional[int] = None) -> Tuple[int, ...]:
    """(tile n, tile m, wavefronts n, wavefronts m, stages, K per stage, workgroups per CU, non-temporal
    weight loads) of the kernel configuration bi_gemm runs for an m x n x k product on the current device."""
    c = _GemmConfig()
    _check("bi_gemm_tile", lib().bi_gemm_tile(lda or k, ldw or k, m, n, k, ctypes.byref(c)))
    return tuple(getattr(c, f) for f, _ in _GemmConfig._fields_)


def gemm_tile(m: int, n: int, k: int, lda: Optional[int] = None, ldw: Optional[int] = None) -> Tuple[int, int]:
    """(weight rows, A rows) of the output tile bi_gemm runs for an m x n x k product on the current device."""
    return gemm_config(m, n, k, lda, ldw)[:2]


def bi_gemm_add(a: torch.Tensor, w: torch.Tensor, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """out = bf16(x + bf16(a w^T)): bi_gemm and bi_add in one kernel (out may be x)."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    _dev(x, "x", torch.bfloat16)
    m, k = a.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if x.shape != (m, n):
        raise ValueError("x must be [m, n]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != (m, n):
        raise ValueError("out shape")
    _check("bi_gemm_add", lib().bi_gemm_add(a.data_ptr(), _rows(a, "a"), w.data_ptr(), _rows(w, "w"),
                                            x.data_ptr(), _rows(x, "x"), out.data_ptr(), _rows(out, "out"),
                                            m, n, k, _stream(stream)))
    return out


def interleave_gate_up(w_gu: torch.Tensor) -> torch.Tensor:
    """The [gate; up] weight [2f, k] with its rows interleaved (gate row j at
    2j, up row j at 2j + 1), the layout bi_gemm_silu_mul reads.  A one-time
    re-layout of a weight (a copy), done when a layer is built."""
    if w_gu.dim() != 2 or w_gu.shape[0] % 2:
        raise ValueError("w_gu must be [2f, k]")
    f, k = w_gu.shape[0] // 2, w_gu.shape[1]
    return w_gu.view(2, f, k).transpose(0, 1).contiguous().view(2 * f, k)


def bi_gemm_silu_mul(a: torch.Tensor, w_gate_up: torch.Tensor, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """out[:, j] = bf16(silu(g_j) * u_j) with g_j, u_j the bf16 products of a with rows 2j and 2j + 1 of
    the interleaved weight (interleave_gate_up): bi_gemm and bi_silu_mul in one kernel."""
    _dev(a, "a", torch.bfloat16)
    _dev(w_gate_up, "w_gate_up", torch.bfloat16)
    m, k = a.shape
    n, k2 = w_gate_up.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if n % 2:
        raise ValueError("w_gate_up must have 2f rows")
    f = n // 2
    if out is None:
        out = torch.empty((m, f), dtype=torch.bfloat16, device=a.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != (m, f):
        raise ValueError("out shape")
    _check("bi_gemm_silu_mul", lib().bi_gemm_silu_mul(a.data_ptr(), _rows(a, "a"), w_gate_up.data_ptr(),
                                                      _rows(w_gate_up, "w_gate_up"), out.data_ptr(),
                                                      _rows(out, "out"), m, f, k, _stream(stream)))
    return out


def alloc_kv_cache(num_pages: int, num_kv_heads: int, head_dim: int, page_size: int = 16,
                   device="cuda", fill: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V caches, each [pages, Hkv, page_size, D] bf16.  The shape only
    sizes the storage: inside a (page, head) block the elements follow the
    tiled order documented in include/bi.h, written by bi_kv_append."""
    k = torch.empty((num_pages, num_kv_heads, page_size, head_dim), dtype=torch.bfloat16, device=device)
    v = torch.empty((num_pages, num_kv_heads, page_size, head_dim), dtype=torch.bfloat16, device=device)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return k, v


def _cache_geom(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _dev(k_cache, "k_cache", torch.bfloat16)
    _dev(v_cache, "v_cache", torch.bfloat16)
    if k_cache.dim() != 4 or not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise ValueError("caches must be contiguous 4-D tensors")
    pages, hkv, ps, d = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [pages, Hkv, page_size, D]")
    return pages, hkv, ps, d


def bi_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                 k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    pages, hkv, ps, d = _cache_geom(k_cache, v_cache)
    _dev(k_new, "k_new", torch.bfloat16)
    _dev(v_new, "v_new", torch.bfloat16)
    _dev(slot_mapping, "slot_mapping", torch.int32)
    t = k_new.shape[0]
    if tuple(k_new.shape) != (t, hkv, d) or v_new.shape != k_new.shape or slot_mapping.shape != (t,):
        raise ValueError("k_new/v_new must be [T, Hkv, D] and slot_mapping [T]")
    ld = _tokens(k_new, "k_new")
    if _tokens(v_new, "v_new") != ld or not slot_mapping.is_contiguous():
        raise ValueError("k_new and v_new need the same token stride; slot_mapping contiguous")
    _check("bi_kv_append", lib().bi_kv_append(k_new.data_ptr(), v_new.data_ptr(), ld, slot_mapping.data_ptr(), t,
                                              k_cache.data_ptr(), v_cache.data_ptr(), pages, hkv, d, ps,
                                              _stream(stream)))


def bi_attn_decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_seq_len: int) -> int:
    return int(lib().bi_attn_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len))


def bi_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Decode attention; returns (out, lse) (lse is None unless a tensor is given)."""
    pages, hkv, ps, d = _cache_geom(k_cache, v_cache)
    _dev(q, "q", torch.bfloat16)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    b, hq, dq = q.shape
    if dq != d:
        raise ValueError("q must be [B, Hq, D]")
    ldq = _tokens(q, "q")
    if block_table.dim() != 2 or block_table.shape[0] != b or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] tensor")
    if seq_lens.shape != (b,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be [B]")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out shape")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != (b, hq) or not lse.is_contiguous():
            raise ValueError("lse must be [B, Hq]")
    need = bi_attn_decode_workspace_bytes(b, hq, d, max_seq_len)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("bi_attn_decode", lib().bi_attn_decode(
        q.data_ptr(), ldq, k_cache.data_ptr(), v_cache.data_ptr(), pages, block_table.data_ptr(),
        block_table.shape[1], seq_lens.data_ptr(), b, int(max_seq_len), hq, hkv, d, ps, float(softmax_scale),
        out.data_ptr(), lse.data_ptr() if lse is not None else None, workspace.data_ptr(), ws_bytes,
        _stream(stream)))
    return out, lse


def bi_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                           softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None):
    """Decode attention with the library's fixed scratch array as its workspace
    (the C entry point allocates nothing).  `out` is required, so this
    wrapper allocates nothing either.  Returns (out, lse)."""
    pages, hkv, ps, d = _cache_geom(k_cache, v_cache)
    _dev(q, "q", torch.bfloat16)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    b, hq, dq = q.shape
    if dq != d:
        raise ValueError("q must be [B, Hq, D]")
    ldq = _tokens(q, "q")
    if block_table.dim() != 2 or block_table.shape[0] != b or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [B, max_pages] tensor")
    if seq_lens.shape != (b,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be [B]")
    _dev(out, "out", torch.bfloat16)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out shape")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != (b, hq) or not lse.is_contiguous():
            raise ValueError("lse must be [B, Hq]")
    _check("bi_attn_decode_noalloc", lib().bi_attn_decode_noalloc(
        q.data_ptr(), ldq, k_cache.data_ptr(), v_cache.data_ptr(), pages, block_table.data_ptr(),
        block_table.shape[1], seq_lens.data_ptr(), b, int(max_seq_len), hq, hkv, d, ps, float(softmax_scale),
        out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(stream)))
    return out, lse


def bi_attn_prefill_workspace_bytes(num_seqs: int) -> int:
    return int(lib().bi_attn_prefill_workspace_bytes(num_seqs))


def bi_attn_prefill(q: torch.Tensor, q_start: torch.Tensor, ctx_lens: torch.Tensor, max_q_len: int,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                    softmax_scale: float, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    order_table: bool = True, stream=None):
    """Chunked-prefill attention; returns (out, lse).  The workspace holds the
    placement order table (allocated here when not given); order_table=False
    passes none, and the kernel ranks the sequences itself."""
    pages, hkv, ps, d = _cache_geom(k_cache, v_cache)
    _dev(q, "q", torch.bfloat16)
    _dev(q_start, "q_start", torch.int32)
    _dev(ctx_lens, "ctx_lens", torch.int32)
    _dev(block_table, "block_table", torch.int32)
    t, hq, dq = q.shape
    s = ctx_lens.shape[0]
    if dq != d:
        raise ValueError("q must be [T, Hq, D]")
    ldq = _tokens(q, "q")
    if q_start.shape != (s + 1,) or not q_start.is_contiguous() or not ctx_lens.is_contiguous():
        raise ValueError("q_start must be [S + 1] and ctx_lens [S]")
    if block_table.dim() != 2 or block_table.shape[0] != s or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous [S, max_pages] tensor")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out shape")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != (t, hq) or not lse.is_contiguous():
            raise ValueError("lse must be [T, Hq]")
    ws_ptr, ws_bytes = None, 0
    if order_table:
        if workspace is None:
            workspace = torch.empty((max(bi_attn_prefill_workspace_bytes(s), 256),), dtype=torch.uint8,
                                    device=q.device)
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check("bi_attn_prefill", lib().bi_attn_prefill(
        q.data_ptr(), ldq, q_start.data_ptr(), ctx_lens.data_ptr(), s, int(max_q_len), k_cache.data_ptr(),
        v_cache.data_ptr(), pages, block_table.data_ptr(), block_table.shape[1], hq, hkv, d, ps,
        float(softmax_scale), out.data_ptr(), lse.data_ptr() if lse is not None else None, ws_ptr, ws_bytes,
        _stream(stream)))
    return out, lse


def bi_log_softmax(logits: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(logits, "logits", torch.float32)
    rows, vocab = logits.shape
    if out is None:
        out = torch.empty((rows, vocab), dtype=torch.float32, device=logits.device)
    _dev(out, "out", torch.float32)
    if out.shape != logits.shape:
        raise ValueError("out shape")
    _check("bi_log_softmax", lib().bi_log_softmax(logits.data_ptr(), _rows(logits, "logits"), out.data_ptr(),
                                                  _rows(out, "out"), rows, vocab, _stream(stream)))
    return out


def moe_workspace_bytes(num_tokens: int, top_k: int, num_experts: int, hidden: int, ffn: int) -> int:
    return int(lib().bi_moe_workspace_bytes(num_tokens, top_k, num_experts, hidden, ffn))


def bi_moe_ffn(x: torch.Tensor, expert_ids: torch.Tensor, expert_weights: torch.Tensor, w_up: torch.Tensor,
               w_down: torch.Tensor, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """x [T, H] bf16; expert_ids [T, k] int32; expert_weights [T, k] fp32;
    w_up [E, F, H] bf16; w_down [E, H, F] bf16 -> y [T, H] bf16."""
    _dev(x, "x", torch.bfloat16)
    _dev(expert_ids, "expert_ids", torch.int32)
    _dev(expert_weights, "expert_weights", torch.float32)
    _dev(w_up, "w_up", torch.bfloat16)
    _dev(w_down, "w_down", torch.bfloat16)
    T, H = x.shape
    E, F, H2 = w_up.shape
    if H2 != H or tuple(w_down.shape) != (E, H, F):
        raise ValueError("w_up must be [E, F, H] and w_down [E, H, F]")
    if expert_ids.dim() != 2 or expert_ids.shape[0] != T or expert_weights.shape != expert_ids.shape:
        raise ValueError("expert_ids / expert_weights must be [T, top_k]")
    for t, name in ((expert_ids, "expert_ids"), (expert_weights, "expert_weights"), (w_up, "w_up"),
                    (w_down, "w_down")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    k = expert_ids.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != (T, H):
        raise ValueError("out shape")
    need = moe_workspace_bytes(T, k, E, H, F)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    _check("bi_moe_ffn", lib().bi_moe_ffn(x.data_ptr(), _rows(x, "x"), expert_ids.data_ptr(),
                                          expert_weights.data_ptr(), T, k, E, w_up.data_ptr(), w_down.data_ptr(),
                                          H, F, out.data_ptr(), _rows(out, "out"), workspace.data_ptr(),
                                          workspace.numel(), _stream(stream)))
    return out


def bi_moe_route(x: torch.Tensor, w_gate: torch.Tensor, top_k: int, logits: Optional[torch.Tensor] = None,
                 expert_ids: Optional[torch.Tensor] = None, expert_weights: Optional[torch.Tensor] = None,
                 stream=None):
    """x [T, H] bf16; w_gate [E, H] bf16 -> (expert_ids [T, top_k] int32,
    expert_weights [T, top_k] fp32, logits [T, E] fp32)."""
    _dev(x, "x", torch.bfloat16)
    _dev(w_gate, "w_gate", torch.bfloat16)
    T, H = x.shape
    E, H2 = w_gate.shape
    if H2 != H or not w_gate.is_contiguous():
        raise ValueError("w_gate must be a contiguous [E, H] tensor")
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    if expert_ids is None:
        expert_ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    if expert_weights is None:
        expert_weights = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    _dev(logits, "logits", torch.float32)
    _dev(expert_ids, "expert_ids", torch.int32)
    _dev(expert_weights, "expert_weights", torch.float32)
    for t, name, shape in ((logits, "logits", (T, E)), (expert_ids, "expert_ids", (T, top_k)),
                           (expert_weights, "expert_weights", (T, top_k))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {shape} tensor")
    _check("bi_moe_route", lib().bi_moe_route(x.data_ptr(), _rows(x, "x"), w_gate.data_ptr(), T, H, E, top_k,
                                              logits.data_ptr(), expert_ids.data_ptr(), expert_weights.data_ptr(),
                                              _stream(stream)))
    return expert_ids, expert_weights, logits


def lm_head_logprobs_workspace_bytes(m: int, n: int) -> int:
    return int(lib().bi_lm_head_logprobs_workspace_bytes(m, n))


def bi_lm_head_logprobs(a: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """out[m, n] = log_softmax_n(sum_k a[m, k] * w[n, k]) in fp32 (GEMM and reduction fused)."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    m, k = a.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _dev(out, "out", torch.float32)
    if out.shape != (m, n):
        raise ValueError("out shape")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != (m,) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous [m] tensor")
    need = lm_head_logprobs_workspace_bytes(m, n)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=a.device)
    _dev(workspace, "workspace", torch.uint8)
    _check("bi_lm_head_logprobs", lib().bi_lm_head_logprobs(
        a.data_ptr(), _rows(a, "a"), w.data_ptr(), _rows(w, "w"), out.data_ptr(), _rows(out, "out"),
        lse.data_ptr() if lse is not None else None, m, n, k, workspace.data_ptr(), workspace.numel(),
        _stream(stream)))
    return out


def lm_head_greedy_workspace_bytes(m: int, n: int) -> int:
    return int(lib().bi_lm_head_greedy_workspace_bytes(m, n))


def bi_lm_head_greedy(a: torch.Tensor, w: torch.Tensor, token: Optional[torch.Tensor] = None,
                      logprob: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None):
    """token[m] = argmax_n (a @ w.T)[m, n] (lowest index on ties) and its fp32
    logprob, without writing the logits.  Returns (token, logprob)."""
    _dev(a, "a", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    m, k = a.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    if token is None:
        token = torch.empty((m,), dtype=torch.int32, device=a.device)
    _dev(token, "token", torch.int32)
    if token.shape != (m,) or not token.is_contiguous():
        raise ValueError("token must be a contiguous [m] tensor")
    if logprob is not None:
        _dev(logprob, "logprob", torch.float32)
        if logprob.shape != (m,) or not logprob.is_contiguous():
            raise ValueError("logprob must be a contiguous [m] tensor")
    need = lm_head_greedy_workspace_bytes(m, n)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=a.device)
    _dev(workspace, "workspace", torch.uint8)
    _check("bi_lm_head_greedy", lib().bi_lm_head_greedy(
        a.data_ptr(), _rows(a, "a"), w.data_ptr(), _rows(w, "w"), token.data_ptr(),
        logprob.data_ptr() if logprob is not None else None, m, n, k, workspace.data_ptr(), workspace.numel(),
        _stream(stream)))
    return token, logprob


def bi_add(x: torch.Tensor, y: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out = bf16(x + y) elementwise over [rows, cols] (out may be x or y)."""
    _dev(x, "x", torch.bfloat16)
    _dev(y, "y", torch.bfloat16)
    if x.dim() != 2 or x.shape != y.shape:
        raise ValueError("x and y must be [rows, cols] of one shape")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != x.shape:
        raise ValueError("out shape")
    rows, cols = x.shape
    _check("bi_add", lib().bi_add(x.data_ptr(), _rows(x, "x"), y.data_ptr(), _rows(y, "y"), out.data_ptr(),
                                  _rows(out, "out"), rows, cols, _stream(stream)))
    return out


def bi_silu_mul(gate_up: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out[i, j] = bf16(silu(gate_up[i, j]) * gate_up[i, f + j]), f = gate_up.shape[1] // 2."""
    _dev(gate_up, "gate_up", torch.bfloat16)
    if gate_up.dim() != 2 or gate_up.shape[1] % 2:
        raise ValueError("gate_up must be [rows, 2f]")
    rows, f = gate_up.shape[0], gate_up.shape[1] // 2
    if out is None:
        out = torch.empty((rows, f), dtype=torch.bfloat16, device=gate_up.device)
    _dev(out, "out", torch.bfloat16)
    if out.shape != (rows, f):
        raise ValueError("out shape")
    _check("bi_silu_mul", lib().bi_silu_mul(gate_up.data_ptr(), _rows(gate_up, "gate_up"), out.data_ptr(),
                                            _rows(out, "out"), rows, f, _stream(stream)))
    return out
