"""bi_attn_decode_noalloc: decode attention whose workspace is the library's
fixed scratch array.  Called through the C-ABI, it must give bitwise the
outputs of bi_attn_decode with a caller-owned workspace, call after call, as
the array keeps what the previous call left in it (here: a large batch that
takes the work-queue path, then a smaller one on the per-chunk path), and
refuse a problem whose workspace would not fit."""
import math

import pytest
import torch

import workloads as W
from _helpers import O, assert_bf16_close, assert_bitwise, assert_f32_close, bi, ensure_lib, f64, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _batch(B, hq, hkv, d, hi, base):
    lens = W.decode_lengths(range(B), base, 1, hi)
    pb = W.allocate_pages(lens, base)
    kc, vc = bi.alloc_kv_cache(pb.num_pages, hkv, d, 16, fill=float("nan"))
    kv = [W.request_kv(r, L, hkv, d, base, device=DEV) for r, L in enumerate(lens)]
    bi.bi_kv_append(torch.cat([k for k, _ in kv]).contiguous(), torch.cat([v for _, v in kv]).contiguous(),
                    pb.slot_mapping.to(DEV), kc, vc)
    q = torch.stack([W.randn_bf16((hq, d), base, "q", r, device=DEV) for r in range(B)])
    return lens, kc, vc, pb.block_table.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV), q, kv


def _both(q, kc, vc, bt, lt, msl, scale):
    B, hq, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, hq), dtype=torch.float32, device=DEV)
    bi.bi_attn_decode_noalloc(q, kc, vc, bt, lt, msl, scale, out, lse=lse)
    ro, rl = bi.bi_attn_decode(q, kc, vc, bt, lt, msl, scale,
                               lse=torch.empty((B, hq), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    return out, lse, ro, rl


def test_noalloc_decode_matches_workspace_decode():
    d, scale = 128, 1.0 / math.sqrt(128)
    # first call: the Qwen3-8B decode workload's full batch (256 sequences of
    # 1..4096 tokens, whole-sequence work queue); second call: 5 sequences of
    # 1..1000 tokens (one wavefront per chunk, then the merge kernel)
    for B, hi, base in ((256, 4096, W.SEED_DECODE), (5, 1000, 41)):
        log_case(f"noalloc decode B={B} max_len={hi}")
        lens, kc, vc, bt, lt, q, kv = _batch(B, 32, 8, d, hi, base)
        msl = max(lens)
        need = bi.bi_attn_decode_workspace_bytes(B, 32, d, msl)
        assert need <= bi.BI_DECODE_SCRATCH_BYTES
        out, lse, ro, rl = _both(q, kc, vc, bt, lt, msl, scale)
        assert_bitwise(out, ro, f"noalloc vs workspace decode, B={B}")
        assert_bitwise(lse, rl, f"noalloc vs workspace lse, B={B}")
        for i in (0, B - 1):
            oo, ol = O.decode_attention(f64(q[i:i + 1]), [f64(kv[i][0])], [f64(kv[i][1])], scale)
            assert_bf16_close(out[i], oo[0], f"noalloc request {i} vs oracle")
            assert_f32_close(lse[i:i + 1], ol, f"noalloc request {i} lse vs oracle")
        # the same call again over what the previous one left in the array
        out2, lse2, _, _ = _both(q, kc, vc, bt, lt, msl, scale)
        assert_bitwise(out2, ro, f"noalloc repeat, B={B}")
        assert_bitwise(lse2, rl, f"noalloc repeat lse, B={B}")


def test_noalloc_decode_refuses_oversized_workspace():
    """A problem whose workspace exceeds the array is refused before any
    launch, and its output is left as it was."""
    d, scale = 128, 1.0 / math.sqrt(128)
    lens, kc, vc, bt, lt, q, _ = _batch(2, 32, 8, d, 300, 43)
    msl = 1 << 20   # 2 x 32 heads x 4096 chunks x 528 bytes > 128 MiB
    assert bi.bi_attn_decode_workspace_bytes(2, 32, d, msl) > bi.BI_DECODE_SCRATCH_BYTES
    out = torch.full_like(q, 3.0)
    with pytest.raises(bi.BiError) as e:
        bi.bi_attn_decode_noalloc(q, kc, vc, bt, lt, msl, scale, out)
    assert e.value.status == bi.BI_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "output touched by a refused call"
