"""bi_rmsnorm on the GPU: parity with the fp64 oracle, closed forms, and the
pages' property (a row's bits do not depend on the batch)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import O, assert_bf16_close, assert_bitwise, bi, ensure_lib, f64, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda"
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _gamma(hidden, base):
    return W.randn_bf16((hidden,), base, "gamma", W.WEIGHTS, std=0.1, mean=1.0)


@pytest.mark.parametrize("hidden,rows", [(512, 1), (512, 3), (512, 8), (4096, 1), (4096, 8), (4096, 64),
                                         (4096, 256), (4096, 2300), (8, 5), (520, 7), (6144, 33), (16384, 4)])
def test_rmsnorm_parity(hidden, rows):
    log_case(f"rmsnorm parity hidden={hidden} rows={rows}")
    base = W.SEED_TINY if hidden == 512 else W.SEED_DECODE
    x = W.rows_for_requests(range(rows), hidden, base)
    g = _gamma(hidden, base)
    y = bi.bi_rmsnorm(x.to(DEV), g.to(DEV), EPS)
    torch.cuda.synchronize()
    ref = O.rmsnorm(f64(x), f64(g), EPS)
    assert_bf16_close(y, ref, f"rmsnorm {hidden}x{rows}")


def test_rmsnorm_closed_forms_on_gpu():
    H = 4096
    ones = torch.ones((3, H), dtype=torch.bfloat16, device=DEV)
    y = bi.bi_rmsnorm(ones, torch.ones(H, dtype=torch.bfloat16, device=DEV), EPS)
    want = O.f64_to_bf16_bits(np.array([1.0 / math.sqrt(1.0 + EPS)])).view(np.int16)[0]
    assert torch.all(y.view(torch.int16).cpu() == int(want))
    z = bi.bi_rmsnorm(torch.zeros((2, H), dtype=torch.bfloat16, device=DEV),
                      torch.ones(H, dtype=torch.bfloat16, device=DEV), EPS)
    assert torch.all(z.view(torch.int16).cpu() == 0)


def test_rmsnorm_in_place_alias():
    x = W.rows_for_requests(range(16), 4096, W.SEED_DECODE).to(DEV)
    g = _gamma(4096, W.SEED_DECODE).to(DEV)
    y = bi.bi_rmsnorm(x, g, EPS)
    x2 = x.clone()
    bi.bi_rmsnorm(x2, g, EPS, out=x2)
    assert_bitwise(x2, y, "in-place rmsnorm")


def test_rmsnorm_batch_invariance():
    hidden = 4096
    g = _gamma(hidden, W.SEED_DECODE).to(DEV)
    ref = None
    for B in (1, 8, 64, 256, 2048):
        for pos in sorted({0, B // 2, B - 1}):
            ids = list(range(1, B))
            ids.insert(pos, 0)                 # request 0 at slot `pos`
            x = W.rows_for_requests(ids, hidden, W.SEED_DECODE, device=DEV)
            y = bi.bi_rmsnorm(x, g, EPS)
            row = y[pos].clone()
            if ref is None:
                ref = row
            assert_bitwise(row, ref, f"rmsnorm request 0 at B={B} slot={pos}")


def test_rmsnorm_run_to_run():
    x = W.rows_for_requests(range(64), 4096, W.SEED_DECODE, device=DEV)
    g = _gamma(4096, W.SEED_DECODE).to(DEV)
    y0 = bi.bi_rmsnorm(x, g, EPS)
    for _ in range(20):
        assert_bitwise(bi.bi_rmsnorm(x, g, EPS), y0, "rmsnorm repeat")


def test_rmsnorm_empty_and_errors():
    g = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    out = bi.bi_rmsnorm(torch.empty((0, 4096), dtype=torch.bfloat16, device=DEV), g, EPS)
    assert out.shape == (0, 4096)
    with pytest.raises(bi.BiError) as e:
        bi.bi_rmsnorm(torch.ones((2, 12), dtype=torch.bfloat16, device=DEV),
                      torch.ones(12, dtype=torch.bfloat16, device=DEV), EPS)
    assert e.value.status == bi.BI_ERR_UNSUPPORTED
