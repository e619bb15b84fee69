"""The library inside a captured HIP graph.  Its calls only enqueue kernels on
the given stream (no allocation, no memset, no host synchronisation) and the
decode work queue resets its own counter on the device at every launch, so a
captured call replays correctly.  Every replay is compared bitwise with the
eager result, with other eager work (which rewrites the same workspace) and
synchronisations between the replays."""
import math

import pytest
import torch

import workloads as W
from _helpers import assert_bitwise, bi, ensure_lib, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _decode_batch(B, hq=32, hkv=8, d=128, base=W.SEED_DECODE):
    lens = W.decode_lengths(range(B), base)
    pb = W.allocate_pages(lens, base)
    kc, vc = bi.alloc_kv_cache(pb.num_pages, hkv, d, 16, DEV, fill=0.0)
    kv = [W.request_kv(r, L, hkv, d, base, device=DEV) for r, L in enumerate(lens)]
    bi.bi_kv_append(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]), pb.slot_mapping.to(DEV), kc, vc)
    q = W.randn_bf16((B, hq, d), base, "q", 0, device=DEV)
    return q, kc, vc, pb.block_table.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def test_decode_capture_replay():
    # B=256: whole-sequence work queue; B=64: chunk groups and the merge kernel;
    # B=8: one wavefront per chunk.  One workspace shared by all of them.
    hq, d = 32, 128
    q, kc, vc, bt, lt = _decode_batch(256)
    ws = torch.empty((bi.bi_attn_decode_workspace_bytes(256, hq, d, 4096),), dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(d)
    for B in (256, 64, 8):
        log_case(f"decode capture/replay B={B}")
        o = torch.empty((B, hq, d), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)

        def call():
            bi.bi_attn_decode(q[:B], kc, vc, bt[:B], lt[:B], 4096, scale, out=o, lse=lse, workspace=ws)

        call()
        torch.cuda.synchronize()
        ref_o, ref_l = o.clone(), lse.clone()
        g = _capture(call)
        other = 256 if B != 256 else 32
        o2 = torch.empty((other, hq, d), dtype=torch.bfloat16, device=DEV)
        for r in range(3):
            # eager work on the same workspace between replays
            bi.bi_attn_decode(q[:other], kc, vc, bt[:other], lt[:other], 4096, scale, out=o2, workspace=ws)
            torch.cuda.synchronize()
            o.fill_(0)
            lse.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert_bitwise(o, ref_o, f"decode B={B} replay {r}")
            assert_bitwise(lse, ref_l, f"decode B={B} lse replay {r}")


def test_gemm_rmsnorm_capture_replay():
    log_case("gemm + rmsnorm capture/replay")
    x = W.rows_for_requests(range(64), 4096, W.SEED_DECODE, device=DEV)
    g1 = W.randn_bf16((4096,), W.SEED_DECODE, "gamma", W.WEIGHTS, std=0.1, mean=1.0, device=DEV)
    w = W.randn_bf16((6144, 4096), W.SEED_DECODE, "w", W.WEIGHTS + 1, std=0.02, device=DEV)
    h = torch.empty_like(x)
    c = torch.empty((64, 6144), dtype=torch.bfloat16, device=DEV)

    def call():
        bi.bi_rmsnorm(x, g1, 1e-6, out=h)
        bi.bi_gemm(h, w, out=c)

    call()
    torch.cuda.synchronize()
    ref = c.clone()
    g = _capture(call)
    for r in range(3):
        bi.bi_gemm(x, w, out=torch.empty_like(c))
        torch.cuda.synchronize()
        c.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(c, ref, f"gemm replay {r}")
