"""The C-ABI library on the CPU host: it loads, exports every function that
include/bi.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os

import pytest

from _helpers import bi, ensure_lib


@pytest.fixture(scope="module")
def lib():
    return ensure_lib()


def test_exports_every_declared_symbol(lib):
    names = bi.header_symbols()
    assert set(names) >= {"bi_rmsnorm", "bi_gemm", "bi_kv_append", "bi_attn_decode", "bi_attn_prefill",
                          "bi_attn_decode_workspace_bytes", "bi_log_softmax", "bi_status_str", "bi_version"}
    for n in names:
        assert hasattr(lib, n), n
        assert n in bi._SIGNATURES, f"{n} has no Python binding"


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(bi.status_str(code), str) and bi.status_str(code)
    assert bi.status_str(-3) == "workspace missing or too small"


def test_host_validation_without_gpu(lib):
    P = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation first
    assert lib.bi_rmsnorm(None, 8, None, 1e-6, None, 8, 4, 8, None) == bi.BI_ERR_INVALID_ARG
    assert lib.bi_rmsnorm(P, 16, P, 1e-6, P, 16, 4, 12, None) == bi.BI_ERR_UNSUPPORTED
    assert lib.bi_rmsnorm(P, 16, P, 1e-6, P, 16, 0, 16, None) == bi.BI_OK          # empty: no-op
    assert lib.bi_rmsnorm(P, 8, P, -1.0, P, 16, 4, 16, None) == bi.BI_ERR_INVALID_ARG
    assert lib.bi_gemm(P, 64, P, 64, P, 64, 0, 4, 4, 48, None) == bi.BI_ERR_UNSUPPORTED   # k % 32
    assert lib.bi_gemm(P, 64, P, 64, P, 64, 7, 4, 4, 64, None) == bi.BI_ERR_INVALID_ARG   # dtype
    assert lib.bi_gemm(P, 32, P, 64, P, 64, 0, 4, 4, 64, None) == bi.BI_ERR_INVALID_ARG   # lda < k
    assert lib.bi_gemm(P, 64, P, 64, P, 64, 0, 0, 4, 64, None) == bi.BI_OK
    # fused epilogues: the GEMM checks, then x / y / out
    assert lib.bi_gemm_add(P, 64, P, 64, P, 64, P, 64, 4, 4, 48, None) == bi.BI_ERR_UNSUPPORTED   # k % 32
    assert lib.bi_gemm_add(P, 64, P, 64, P, 12, P, 64, 4, 16, 64, None) == bi.BI_ERR_INVALID_ARG  # ldx < n
    assert lib.bi_gemm_add(P, 64, P, 64, P, 64, P, 72, 4, 16, 64, None) == bi.BI_ERR_INVALID_ARG  # y = x, ldy != ldx
    assert lib.bi_gemm_add(P, 64, P, 64, None, 64, P, 64, 4, 16, 64, None) == bi.BI_ERR_INVALID_ARG
    assert lib.bi_gemm_add(P, 64, P, 64, P, 64, P, 64, 0, 16, 64, None) == bi.BI_OK
    assert lib.bi_gemm_silu_mul(P, 64, P, 64, P, 16, 4, 16, 48, None) == bi.BI_ERR_UNSUPPORTED    # k % 32
    assert lib.bi_gemm_silu_mul(P, 64, P, 64, P, 8, 4, 16, 64, None) == bi.BI_ERR_INVALID_ARG     # ldo < f
    assert lib.bi_gemm_silu_mul(P, 64, P, 64, P, 20, 4, 16, 64, None) == bi.BI_ERR_INVALID_ARG    # ldo % 8
    assert lib.bi_gemm_silu_mul(P, 64, P, 64, P, 16, 4, (1 << 29) + 1, 64, None) == bi.BI_ERR_UNSUPPORTED
    assert lib.bi_gemm_silu_mul(P, 64, P, 64, P, 16, 4, 0, 64, None) == bi.BI_OK
    # MoE: hidden not a multiple of 32, missing workspace, empty batch
    moe = lambda T, H, ws, nbytes: lib.bi_moe_ffn(P, H, P, P, T, 8, 128, P, P, H, 1536, P, H, ws, nbytes, None)
    assert moe(4, 4016, P, 1 << 30) == bi.BI_ERR_UNSUPPORTED
    assert moe(4, 4096, None, 1 << 30) == bi.BI_ERR_WORKSPACE
    assert moe(4, 4096, ctypes.c_void_p(256), 16) == bi.BI_ERR_WORKSPACE
    assert moe(0, 4096, None, 0) == bi.BI_OK
    assert lib.bi_moe_workspace_bytes(2048, 8, 128, 4096, 1536) >= 2048 * 8 * (2 * 1536 + 4 * 4096)
    # MoE router: top_k above the experts, too many experts, hidden not a multiple of 32, empty batch
    route = lambda T, H, E, k: lib.bi_moe_route(P, H, P, T, H, E, k, P, P, P, None)
    assert route(4, 4096, 8, 9) == bi.BI_ERR_INVALID_ARG
    assert route(4, 4096, 2048, 8) == bi.BI_ERR_UNSUPPORTED
    assert route(4, 4096, 128, 65) == bi.BI_ERR_UNSUPPORTED
    assert route(4, 4016, 128, 8) == bi.BI_ERR_UNSUPPORTED
    assert route(4, 4096, 128, 0) == bi.BI_ERR_INVALID_ARG
    assert route(0, 4096, 128, 8) == bi.BI_OK
    assert lib.bi_moe_route(None, 4096, P, 4, 4096, 128, 8, P, P, P, None) == bi.BI_ERR_INVALID_ARG
    # a slice of W or A spanning 2^31 bytes cannot be addressed by one buffer resource: at
    # k = 64 (a multiple of 64, not of 128) the rule's candidates read at least 32-row
    # slices of W and 16-row slices of A, so no tile fits these strides
    assert lib.bi_gemm(P, 64, P, 1 << 26, P, 64, 0, 65, 4, 64, None) == bi.BI_ERR_UNSUPPORTED
    assert lib.bi_gemm(P, 64, P, 1 << 26, P, 64, 0, 4, 4, 64, None) == bi.BI_ERR_UNSUPPORTED
    assert lib.bi_gemm(P, 1 << 27, P, 64, P, 64, 0, 4, 4, 64, None) == bi.BI_ERR_UNSUPPORTED
    # a weight of >= 32768 rows runs the 128 x 256 tile: 128 W rows must span < 2^31 bytes
    assert lib.bi_gemm(P, 64, P, 9_000_000, P, 1 << 15, 0, 4, 1 << 15, 64, None) == bi.BI_ERR_UNSUPPORTED
    # decode: head_dim 96, group size 3, page size 12, missing workspace
    args = dict(q=P, kc=P, vc=P, pages=8, bt=P, mp=4, lens=P, b=2, msl=64, hq=32, hkv=8, d=128, ps=16)

    def dec(**kw):
        a = dict(args, **kw)
        return lib.bi_attn_decode(a["q"], a.get("ldq", 4096), a["kc"], a["vc"], a["pages"], a["bt"], a["mp"], a["lens"], a["b"],
                                  a["msl"], a["hq"], a["hkv"], a["d"], a["ps"], 0.1, P, None,
                                  a.get("ws", P), a.get("wsb", 1 << 30), None)

    assert dec(d=96) == bi.BI_ERR_UNSUPPORTED
    assert dec(hq=24) == bi.BI_ERR_UNSUPPORTED
    assert dec(hq=30) == bi.BI_ERR_INVALID_ARG
    assert dec(ps=12) == bi.BI_ERR_UNSUPPORTED
    assert dec(ws=None) == bi.BI_ERR_WORKSPACE
    assert dec(wsb=100) == bi.BI_ERR_WORKSPACE
    assert dec(b=0) == bi.BI_OK
    assert dec(ldq=4000) == bi.BI_ERR_INVALID_ARG
    # prefill: a workspace that is short or misaligned is refused before any launch
    pre = lambda ws, nbytes: lib.bi_attn_prefill(P, 4096, P, P, 40, 64, P, P, 8, P, 4, 32, 8, 128, 16, 0.1, P, None,
                                                 ws, nbytes, None)
    assert lib.bi_attn_prefill_workspace_bytes(40) >= 160
    assert pre(P, 100) == bi.BI_ERR_WORKSPACE
    assert pre(ctypes.c_void_p(24), 1 << 20) == bi.BI_ERR_WORKSPACE
    assert lib.bi_log_softmax(P, 6, P, 8, 2, 6, None) == bi.BI_ERR_UNSUPPORTED
    # fused lm_head + log_softmax: n % 4, k % 32, short or missing or misaligned workspace, ldo, empty batch
    W256 = ctypes.c_void_p(256)
    lmh = lambda m, n, k, ldo, ws, nbytes: lib.bi_lm_head_logprobs(P, k, P, k, P, ldo, None, m, n, k, ws, nbytes, None)
    assert lmh(2, 1026, 64, 1028, W256, 1 << 30) == bi.BI_ERR_UNSUPPORTED
    assert lmh(2, 1024, 48, 1024, W256, 1 << 30) == bi.BI_ERR_UNSUPPORTED
    assert lmh(2, 1024, 64, 1024, None, 1 << 30) == bi.BI_ERR_WORKSPACE
    assert lmh(2, 1024, 64, 1024, ctypes.c_void_p(272), 1 << 30) == bi.BI_ERR_WORKSPACE
    assert lmh(2, 1024, 64, 1024, W256, 16) == bi.BI_ERR_WORKSPACE
    assert lmh(2, 1024, 64, 1022, W256, 1 << 30) == bi.BI_ERR_INVALID_ARG
    assert lmh(0, 1024, 64, 1024, None, 0) == bi.BI_OK
    # greedy lm_head: k % 32, misaligned token, short or missing or misaligned workspace, empty batch
    T4 = ctypes.c_void_p(64)
    gr = lambda m, n, k, tok, ws, nbytes: lib.bi_lm_head_greedy(P, k, P, k, tok, None, m, n, k, ws, nbytes, None)
    assert gr(2, 1026, 48, T4, W256, 1 << 30) == bi.BI_ERR_UNSUPPORTED
    assert gr(2, 1026, 64, ctypes.c_void_p(66), W256, 1 << 30) == bi.BI_ERR_INVALID_ARG
    assert gr(2, 1026, 64, None, W256, 1 << 30) == bi.BI_ERR_INVALID_ARG
    assert gr(2, 1026, 64, T4, None, 1 << 30) == bi.BI_ERR_WORKSPACE
    assert gr(2, 1026, 64, T4, ctypes.c_void_p(272), 1 << 30) == bi.BI_ERR_WORKSPACE
    assert gr(2, 1026, 64, T4, W256, 16) == bi.BI_ERR_WORKSPACE
    assert gr(0, 1026, 64, None, None, 0) == bi.BI_OK
    assert lib.bi_kv_append(P, P, 640, P, 3, P, P, 4, 8, 80, 16, None) == bi.BI_ERR_UNSUPPORTED
    assert lib.bi_kv_append(P, P, 1000, P, 3, P, P, 4, 8, 128, 16, None) == bi.BI_ERR_INVALID_ARG


def test_workspace_size_formula(lib):
    # one (D + 4)-float record per (sequence, q head, 256-token chunk), rounded to 256 bytes, then the
    # work queue: a 16-byte header and two int32 entries per (sequence, chunk), rounded to 256 bytes
    r256 = lambda x: (x + 255) // 256 * 256
    n = bi.bi_attn_decode_workspace_bytes(3, 32, 128, 1000)
    assert n == r256(r256(3 * 32 * 4 * (128 + 4) * 4) + 16 + 8 * 3 * 4)
    assert bi.bi_attn_decode_workspace_bytes(1, 1, 64, 256) == r256(r256(68 * 4) + 16 + 8)
    assert bi.bi_attn_decode_workspace_bytes(256, 32, 128, 4096) == r256(r256(256 * 32 * 16 * 132 * 4) + 16 + 8 * 256 * 16)
    # one (max, sum) pair of fp32 per (row, n-tile), rounded to 256 bytes; the
    # n-tile is the GEMM's: 64 columns below 32768, 128 from 32768 on
    assert bi.lm_head_logprobs_workspace_bytes(2048, 151936) == 2048 * 1187 * 8
    assert bi.lm_head_logprobs_workspace_bytes(5, 32764) == (5 * 512 * 8 + 255) // 256 * 256
    assert bi.lm_head_logprobs_workspace_bytes(5, 32768) == (5 * 256 * 8 + 255) // 256 * 256
    assert bi.lm_head_logprobs_workspace_bytes(3, 100) == 256
    # greedy: (max, sum, index) of 12 bytes per (row, n-tile), rounded to 256 bytes
    assert bi.lm_head_greedy_workspace_bytes(2048, 151936) == (2048 * 1187 * 12 + 255) // 256 * 256
    assert bi.lm_head_greedy_workspace_bytes(3, 18992) == (3 * 297 * 12 + 255) // 256 * 256
    assert bi.lm_head_greedy_workspace_bytes(3, 100) == 256


def test_adaptive_library_exports_its_header():
    """libbi_adaptive.so (the shape-adaptive comparators) loads and exports
    every function include/bi_adaptive.h declares."""
    import re
    from invariant_bi_rmsnorm_02_amd import adaptive as A
    text = open(os.path.join(os.path.dirname(bi.HEADER), "bi_adaptive.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:int32_t|size_t|bi_status)\s+(bia_\w+)\s*\(", text, re.M)))
    assert len(names) == 9
    lib = A.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert A.gemm_splits(1, 6144, 4096) > 1 and A.gemm_splits(2300, 6144, 4096) == 1
    assert A.decode_split_keys(1, 8, 4096, 16) == 64 and A.decode_split_keys(256, 8, 4096, 16) == 512
    assert A.decode_split_keys(4, 8, 4096, 16) == 256 and A.decode_split_keys(1, 8, 100, 256) == 256
    assert lib.bia_gemm(None, 64, None, 64, None, 64, 4, 4, 64, None, 0, None) == bi.BI_ERR_INVALID_ARG
