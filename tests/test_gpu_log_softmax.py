"""bi_log_softmax on the GPU: parity (fp32 max abs err <= 1e-3), closed forms,
and a token's logprobs bitwise across batch compositions."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import O, assert_bitwise, assert_f32_close, bi, ensure_lib, f64, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda"
V = 151936


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _logits(ids, vocab=V, scale=4.0):
    return torch.stack([torch.randn(vocab, generator=W.gen(W.SEED_MOE, "logits", r)) * scale for r in ids])


@pytest.mark.parametrize("rows,vocab", [(1, V), (3, V), (8, 1024), (5, 4), (2, 100004)])
def test_log_softmax_parity(rows, vocab):
    log_case(f"log_softmax parity rows={rows} vocab={vocab}")
    z = _logits(range(rows), vocab)
    lp = bi.bi_log_softmax(z.to(DEV))
    assert_f32_close(lp, O.log_softmax(f64(z)), f"log_softmax {rows}x{vocab}")


def test_log_softmax_closed_forms():
    z = torch.full((2, V), 3.25, device=DEV)
    assert_f32_close(bi.bi_log_softmax(z), np.full((2, V), -math.log(V)), "constant logits")
    z2 = torch.tensor([[2.0, -1.0, -1e30, -1e30]], device=DEV)
    lp = bi.bi_log_softmax(z2)
    assert abs(lp[0, 0].item() + math.log1p(math.exp(-3.0))) < 1e-6


def test_log_softmax_batch_invariance():
    ref = None
    for T in (1, 64, 512, 2048):
        for pos in sorted({0, T // 2, T - 1}):
            ids = list(range(1, T))
            ids.insert(pos, 0)
            z = _logits(ids).to(DEV)
            row = bi.bi_log_softmax(z)[pos].clone()
            if ref is None:
                ref = row
            assert_bitwise(row, ref, f"token 0 logprobs at T={T} slot={pos}")


def test_log_softmax_in_place():
    z = _logits(range(4)).to(DEV)
    ref = bi.bi_log_softmax(z)
    bi.bi_log_softmax(z, out=z)
    assert_bitwise(z, ref, "in place")
