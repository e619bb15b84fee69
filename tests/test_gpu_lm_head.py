"""bi_lm_head_logprobs on the GPU (lm_head GEMM with log_softmax fused into its
epilogue): parity with the oracle's log_softmax of the oracle's GEMM (fp32
max abs err <= 1e-3), closed forms, a token's logprobs bitwise across batch
compositions, and agreement with the two-call path to rounding."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import O, assert_bitwise, assert_f32_close, bi, ensure_lib, f64, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda"
V = 151936
K = 4096


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _weights(n, k=K):
    return W.randn_bf16((n, k), W.SEED_MOE, "w", W.WEIGHTS, std=0.02, device=DEV)


def _ref(a, w):
    """Oracle logprobs and lse (= z - logprob, read off column 0)."""
    z = O.gemm(f64(a), f64(w))
    lp = O.log_softmax(z)
    return lp, z[:, 0] - lp[:, 0]


@pytest.mark.parametrize("m,n,k", [(1, 1024, 256), (3, 2052, 256), (70, 2052, 512), (5, V // 8, K),
                                   (300, 32900, 256)])
def test_lm_head_logprobs_parity(m, n, k):
    log_case(f"lm_head logprobs parity m={m} n={n} k={k}")
    a = W.rows_for_requests(range(m), k, W.SEED_MOE, device=DEV)
    w = _weights(n, k)
    lse = torch.empty(m, dtype=torch.float32, device=DEV)
    lp = bi.bi_lm_head_logprobs(a, w, lse=lse)
    ref_lp, ref_lse = _ref(a, w)
    assert_f32_close(lp, ref_lp, f"logprobs {m}x{n}x{k}")
    assert_f32_close(lse, ref_lse, f"lse {m}x{n}x{k}")


def test_lm_head_logprobs_full_vocab():
    log_case("lm_head logprobs full vocab T=1")
    a = W.rows_for_requests([0], K, W.SEED_MOE, device=DEV)
    w = _weights(V)
    lp = bi.bi_lm_head_logprobs(a, w)
    assert_f32_close(lp, _ref(a, w)[0], "logprobs 1x151936x4096")
    # probabilities sum to one
    assert abs(float(torch.exp(lp.double()).sum()) - 1.0) < 1e-4


def test_lm_head_logprobs_closed_forms():
    a = W.rows_for_requests(range(2), 256, W.SEED_MOE, device=DEV)
    w = torch.zeros((4096, 256), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(2, dtype=torch.float32, device=DEV)
    lp = bi.bi_lm_head_logprobs(a, w, lse=lse)
    assert_f32_close(lp, np.full((2, 4096), -math.log(4096)), "zero weights: uniform")
    assert_f32_close(lse, np.full(2, math.log(4096)), "zero weights: lse = log n")
    # one-hot rows of A select one column of W: z = w[:, j]
    a1 = torch.zeros((1, 256), dtype=torch.bfloat16, device=DEV)
    a1[0, 7] = 1.0
    w1 = _weights(1024, 256)
    z = f64(w1)[:, 7][None, :]
    assert_f32_close(bi.bi_lm_head_logprobs(a1, w1), O.log_softmax(z), "one-hot row")


def test_lm_head_logprobs_batch_invariance():
    n = V // 8
    w = _weights(n)
    ref = None
    ws = None
    for T in (1, 17, 64, 512):
        for pos in sorted({0, T // 3, T - 1}):
            ids = list(range(1, T))
            ids.insert(pos, 0)
            a = W.rows_for_requests(ids, K, W.SEED_MOE, device=DEV)
            need = bi.lm_head_logprobs_workspace_bytes(T, n)
            if ws is None or ws.numel() < need:
                ws = torch.empty(need, dtype=torch.uint8, device=DEV)
            row = bi.bi_lm_head_logprobs(a, w, workspace=ws)[pos].clone()
            if ref is None:
                ref = row
            assert_bitwise(row, ref, f"token 0 logprobs at T={T} slot={pos}")


def test_lm_head_full_vocab_batch_invariance():
    """The lm_head at the workload's size (4096 -> 151936): token 0's logprobs
    row, greedy token and token logprob bitwise the same at T = 1, 17, 64, 511
    (128 x 256 GEMM tile), 512, 2048 (256 x 256 tile) and shuffled slots; the
    per-row reduction records do not depend on the tile, and a tile's 16-row
    blocks past its last row (skipped in the epilogue) change nothing."""
    w = _weights(V)
    ref = gref = None
    for T, pos in ((1, 0), (17, 16), (64, 50), (511, 510), (512, 0), (2048, 1500)):
        log_case(f"full-vocab lm_head invariance T={T} slot={pos}")
        ids = list(range(1, T))
        ids.insert(pos, 0)
        a = W.rows_for_requests(ids, K, W.SEED_MOE, device=DEV)
        row = bi.bi_lm_head_logprobs(a, w)[pos].clone()
        tok, lp = bi.bi_lm_head_greedy(a, w, logprob=torch.empty(T, dtype=torch.float32, device=DEV))
        got = (int(tok[pos]), lp[pos].clone())
        torch.cuda.empty_cache()
        if ref is None:
            ref, gref = row, got
        assert_bitwise(row, ref, f"token 0 logprobs at T={T} slot={pos}")
        assert got[0] == gref[0], f"greedy token of request 0 at T={T} slot={pos}"
        assert_bitwise(got[1], gref[1], f"greedy logprob of request 0 at T={T} slot={pos}")
    assert_bitwise(ref[gref[0]:gref[0] + 1], gref[1].reshape(1), "greedy logprob == logprobs row at the token")


def test_lm_head_logprobs_matches_two_calls():
    """Same mathematics as bi_gemm (fp32) + bi_log_softmax; a different fixed
    reduction tree for lse, so equal to rounding, not to the bit."""
    a = W.rows_for_requests(range(6), K, W.SEED_MOE, device=DEV)
    w = _weights(V // 8)
    fused = bi.bi_lm_head_logprobs(a, w)
    two = bi.bi_log_softmax(bi.bi_gemm(a, w, out_dtype=torch.float32))
    assert float((fused - two).abs().max()) < 1e-4


def test_lm_head_logprobs_workspace_reuse_and_errors():
    w = _weights(2052, 256)
    a_big = W.rows_for_requests(range(33), 256, W.SEED_MOE, device=DEV)
    a_small = W.rows_for_requests(range(5), 256, W.SEED_MOE, device=DEV)
    ws = torch.full((bi.lm_head_logprobs_workspace_bytes(33, 2052),), 0x7f, dtype=torch.uint8, device=DEV)
    bi.bi_lm_head_logprobs(a_big, w, workspace=ws)
    small = bi.bi_lm_head_logprobs(a_small, w, workspace=ws)   # stale pairs of the bigger call in the workspace
    assert_bitwise(small, bi.bi_lm_head_logprobs(a_small, w), "workspace contents on entry do not matter")
    out = torch.full((5, 2052), 7.0, device=DEV)
    with pytest.raises(bi.BiError) as e:
        bi.bi_lm_head_logprobs(a_small, w, out=out, workspace=ws[:64])
    assert e.value.status == bi.BI_ERR_WORKSPACE
    assert bool((out == 7.0).all()), "nothing written on error"


# ---------------------------------------------------------------- greedy sampling

@pytest.mark.parametrize("m,n,k", [(1, 1024, 256), (3, 2053, 256), (70, 2052, 512), (5, V // 8, K), (1, V, K),
                                   (37, 32901, 256)])
def test_lm_head_greedy_parity(m, n, k):
    """The token is the argmax (lowest index on ties) of the library's own fp32
    logits - the decision taken in the kernel's precision - and its logprob is
    bitwise the logprobs path's value at that token; where the oracle's top two
    logits are clearly apart its argmax agrees too."""
    log_case(f"lm_head greedy parity m={m} n={n} k={k}")
    a = W.rows_for_requests(range(m), k, W.SEED_MOE, device=DEV)
    w = _weights(n, k)
    tok, lp = bi.bi_lm_head_greedy(a, w, logprob=torch.empty(m, dtype=torch.float32, device=DEV))
    z = bi.bi_gemm(a, w, out_dtype=torch.float32).cpu().numpy()
    assert tok.cpu().numpy().tolist() == np.argmax(z, axis=1).tolist(), "token = argmax of the fp32 logits"
    if n % 4 == 0:
        full = bi.bi_lm_head_logprobs(a, w)
        picked = full[torch.arange(m, device=DEV), tok.long()]
        assert_bitwise(lp, picked, "greedy logprob vs logprobs path at the token")
    zo = O.gemm(f64(a), f64(w))
    top2 = np.sort(zo, axis=1)[:, -2:]
    clear = (top2[:, 1] - top2[:, 0]) > 1e-3
    ref_tok = np.argmax(zo, axis=1)
    assert (tok.cpu().numpy()[clear] == ref_tok[clear]).all(), "oracle argmax where the top two are apart"
    ref_lp = O.log_softmax(zo)[np.arange(m), tok.cpu().numpy()]
    assert_f32_close(lp, ref_lp, "greedy logprob vs oracle")


def test_lm_head_greedy_ties_and_closed_forms():
    # equal logits at columns 5, 700 and 1500 (identical weight rows), larger than the rest: the lowest wins
    a = torch.zeros((2, 256), dtype=torch.bfloat16, device=DEV)
    a[:, 0] = 1.0
    w = _weights(2048, 256) * 0.5
    for j in (1500, 700, 5):
        w[j] = 0.0
        w[j, 0] = 3.0
    tok, lp = bi.bi_lm_head_greedy(a, w, logprob=torch.empty(2, dtype=torch.float32, device=DEV))
    assert tok.tolist() == [5, 5]
    # all logits equal (zero weights): token 0, logprob -ln n
    wz = torch.zeros((4100, 256), dtype=torch.bfloat16, device=DEV)
    tok, lp = bi.bi_lm_head_greedy(a, wz, logprob=torch.empty(2, dtype=torch.float32, device=DEV))
    assert tok.tolist() == [0, 0]
    assert_f32_close(lp, np.full(2, -math.log(4100)), "zero weights: logprob = -ln n")
    # the maximum in the ragged last tile
    w2 = _weights(2053, 256) * 0.5
    w2[2052] = 0.0
    w2[2052, 0] = 3.0
    assert bi.bi_lm_head_greedy(a, w2)[0].tolist() == [2052, 2052]


def test_lm_head_greedy_batch_invariance_and_workspace():
    n = V // 8
    w = _weights(n)
    ref = None
    ws = torch.full((bi.lm_head_greedy_workspace_bytes(512, n),), 0x7f, dtype=torch.uint8, device=DEV)
    for T in (1, 64, 512):
        for pos in sorted({0, T // 3, T - 1}):
            ids = list(range(1, T))
            ids.insert(pos, 0)
            a = W.rows_for_requests(ids, K, W.SEED_MOE, device=DEV)
            tok, lp = bi.bi_lm_head_greedy(a, w, logprob=torch.empty(T, dtype=torch.float32, device=DEV),
                                          workspace=ws)
            got = (int(tok[pos]), lp[pos].clone())
            if ref is None:
                ref = got
            assert got[0] == ref[0], f"token of request 0 at T={T} slot={pos}"
            assert_bitwise(got[1], ref[1], f"logprob of request 0 at T={T} slot={pos}")
    with pytest.raises(bi.BiError) as e:
        bi.bi_lm_head_greedy(W.rows_for_requests(range(4), K, W.SEED_MOE, device=DEV), w, workspace=ws[:64])
    assert e.value.status == bi.BI_ERR_WORKSPACE


def test_lm_head_tile_switch_edge():
    """Rows shared by T = 511 (128 x 256 tile) and T = 512 (256 x 256 tile):
    bitwise equal logprobs, lse and greedy results, on a vocabulary with a
    ragged last record (32768 + 200 columns: the big tile's last n-tile holds
    one partial record and one past the end)."""
    n = 32768 + 200
    w = _weights(n, 512)
    a = W.rows_for_requests(range(512), 512, W.SEED_MOE, device=DEV)
    lse_lo = torch.empty(511, dtype=torch.float32, device=DEV)
    lse_hi = torch.empty(512, dtype=torch.float32, device=DEV)
    lo = bi.bi_lm_head_logprobs(a[:511].contiguous(), w, lse=lse_lo)
    hi = bi.bi_lm_head_logprobs(a, w, lse=lse_hi)
    assert_bitwise(hi[:511], lo, "logprobs rows at T=511 vs T=512")
    assert_bitwise(lse_hi[:511], lse_lo, "lse at T=511 vs T=512")
    t_lo, p_lo = bi.bi_lm_head_greedy(a[:511].contiguous(), w, logprob=torch.empty(511, dtype=torch.float32, device=DEV))
    t_hi, p_hi = bi.bi_lm_head_greedy(a, w, logprob=torch.empty(512, dtype=torch.float32, device=DEV))
    assert_bitwise(t_hi[:511], t_lo, "greedy tokens at T=511 vs T=512")
    assert_bitwise(p_hi[:511], p_lo, "greedy logprobs at T=511 vs T=512")
    ref_lp, ref_lse = _ref(a[::97], w)
    assert_f32_close(hi[::97], ref_lp, "logprobs (big tile) vs oracle")
    assert_f32_close(lse_hi[::97], ref_lse, "lse (big tile) vs oracle")
    z = bi.bi_gemm(a, w, out_dtype=torch.float32)
    zlo = bi.bi_gemm(a[:511].contiguous(), w, out_dtype=torch.float32)
    assert_bitwise(z[:511], zlo, "fp32 logits at T=511 vs T=512")
