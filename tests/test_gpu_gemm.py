"""bi_gemm on the GPU: exact integer pins, parity with the fp64 oracle at the
workload shapes, and the pages' property (row m's bits do not depend on the
other rows of A, on M, or on the row's position)."""
import numpy as np
import pytest
import torch

import workloads as W
from _helpers import O, assert_bf16_close, assert_bitwise, assert_f32_close, bi, ensure_lib, f64, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _int_bf16(shape, seed, lo=-4, hi=4):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("m,n,k", [(1, 1024, 512), (8, 1024, 512), (130, 257, 4096), (300, 136, 96),
                                   (17, 40, 32)])
def test_gemm_integer_exact(m, n, k):
    # Products and partial sums are integers below 2^24, so fp32 accumulation is
    # exact in any order; the bf16 result must be the oracle rounded once (RNE).
    log_case(f"gemm integer exact m={m} n={n} k={k}")
    a, w = _int_bf16((m, k), 1), _int_bf16((n, k), 2)
    ref = O.gemm(f64(a), f64(w))
    c16 = bi.bi_gemm(a.to(DEV), w.to(DEV))
    c32 = bi.bi_gemm(a.to(DEV), w.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = torch.from_numpy(O.f64_to_bf16_bits(ref).view(np.int16))
    assert torch.equal(c16.view(torch.int16).cpu(), want)
    assert np.array_equal(f64(c32), ref)


def test_gemm_bf16_output_is_rne_of_fp32_output():
    """The bf16 epilogue (gfx950's v_cvt_pk_bf16_f32) rounds the same fp32
    accumulator the fp32 epilogue stores, once, to nearest with ties to even:
    bitwise equal to the oracle's RNE encoder applied to the fp32 output, over
    1.5 M values spanning many binades (inputs scaled by 2^-20 .. 2^20 per row)."""
    m, n, k = 256, 6144, 256
    a = W.randn_bf16((m, k), W.SEED_DECODE, "x", 4242)
    scale = torch.pow(2.0, torch.linspace(-20, 20, m)).to(torch.bfloat16).unsqueeze(1)
    a = (a * scale).to(torch.bfloat16)
    w = W.randn_bf16((n, k), W.SEED_DECODE, "w", 4243)
    c32 = bi.bi_gemm(a.to(DEV), w.to(DEV), out_dtype=torch.float32)
    c16 = bi.bi_gemm(a.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    want = torch.from_numpy(O.f64_to_bf16_bits(c32.cpu().double().numpy()).view(np.int16))
    assert torch.equal(c16.cpu().view(torch.int16), want)


def test_gemm_identity_and_selector():
    k = 256
    a = W.randn_bf16((37, k), 0, "x", 7)
    eye = torch.eye(k, dtype=torch.bfloat16)
    c = bi.bi_gemm(a.to(DEV), eye.to(DEV))
    assert_bitwise(c.cpu(), a, "A @ I")
    w = W.randn_bf16((100, k), 0, "w", 8)
    sel = torch.zeros((2, k), dtype=torch.bfloat16)
    sel[0, 5] = 1
    sel[1, 200] = 1
    cs = bi.bi_gemm(sel.to(DEV), w.to(DEV)).cpu()
    assert_bitwise(cs[0], w[:, 5].contiguous(), "selector row 0")
    assert_bitwise(cs[1], w[:, 200].contiguous(), "selector row 1")


SHAPES = [
    ("tiny 512->1024", 512, 1024, W.SEED_TINY, 1.0),
    ("qkv 4096->6144", 4096, 6144, W.SEED_DECODE, 0.02),
    ("up 4096->12288", 4096, 12288, W.SEED_DECODE, 0.02),
    ("down 12288->4096", 12288, 4096, W.SEED_DECODE, 0.02),
]


@pytest.mark.parametrize("name,k,n,base,wstd", SHAPES)
@pytest.mark.parametrize("m", [1, 3, 8, 64, 256])
def test_gemm_parity_workload_shapes(name, k, n, base, wstd, m):
    if name.startswith("tiny") and m > 8:
        pytest.skip("tiny workload uses B in {1, 3, 8}")
    log_case(f"gemm parity {name} m={m}")
    w = W.randn_bf16((n, k), base, "w", W.WEIGHTS + k, std=wstd, device=DEV)
    a = W.rows_for_requests(range(m), k, base, device=DEV)
    c = bi.bi_gemm(a, w)
    torch.cuda.synchronize()
    ref = O.gemm(f64(a), f64(w))
    assert_bf16_close(c, ref, f"{name} m={m}")


def test_gemm_parity_large_m_sampled_rows():
    # The mixed prefill+decode batch: M = 2048 + decode rows; check sampled rows.
    m, k, n = 2300, 4096, 6144
    log_case(f"gemm parity large m={m}")
    w = W.randn_bf16((n, k), W.SEED_MIXED, "w", W.WEIGHTS, std=0.02, device=DEV)
    a = W.rows_for_requests(range(m), k, W.SEED_MIXED, device=DEV)
    c = bi.bi_gemm(a, w)
    rows = [0, 1, 127, 128, 1000, 2047, 2048, 2299]
    ref = O.gemm(f64(a[rows]), f64(w))
    assert_bf16_close(c[rows], ref, "large m sampled rows")


def test_gemm_ragged_tails():
    for (m, n, k) in [(129, 131, 96), (5, 1000, 160), (255, 8, 32), (1, 136, 4128)]:
        log_case(f"gemm ragged m={m} n={n} k={k}")
        a = W.randn_bf16((m, k), 9, "x", m)
        w = W.randn_bf16((n, k), 9, "w", n, std=0.05)
        c = bi.bi_gemm(a.to(DEV), w.to(DEV))
        c32 = bi.bi_gemm(a.to(DEV), w.to(DEV), out_dtype=torch.float32)
        ref = O.gemm(f64(a), f64(w))
        assert_bf16_close(c, ref, f"ragged {m}x{n}x{k}")
        assert_f32_close(c32, ref, f"ragged fp32 {m}x{n}x{k}")


def test_gemm_strided_operands():
    a_full = W.randn_bf16((40, 256 + 64), 9, "x", 1).to(DEV)
    w_full = W.randn_bf16((72, 256 + 32), 9, "w", 1).to(DEV)
    out_full = torch.zeros((40, 72 + 24), dtype=torch.bfloat16, device=DEV)
    a, w, out = a_full[:, :256], w_full[:, :256], out_full[:, :72]
    bi.bi_gemm(a, w, out=out)
    ref = O.gemm(f64(a), f64(w))
    assert_bf16_close(out, ref, "strided")
    assert torch.all(out_full[:, 72:] == 0)


@pytest.mark.parametrize("k,n", [(512, 1024), (4096, 6144), (12288, 4096)])
def test_gemm_batch_invariance(k, n):
    w = W.randn_bf16((n, k), W.SEED_DECODE, "w", W.WEIGHTS + k, std=0.02, device=DEV)
    ref = None
    for m in (1, 3, 8, 64, 256, 2051):
        for pos in sorted({0, m // 2, m - 1}):
            ids = list(range(1, m))
            ids.insert(pos, 0)
            a = W.rows_for_requests(ids, k, W.SEED_DECODE, device=DEV)
            row = bi.bi_gemm(a, w)[pos].clone()
            if ref is None:
                ref = row
            assert_bitwise(row, ref, f"gemm k={k} n={n}: request 0 at M={m} slot={pos}")


def test_gemm_fp32_lm_head_invariance():
    # lm_head-shaped fp32 output on a vocab slice; token 0's logits at T in {1, 64, 512}.
    k, n = 4096, 151936 // 8
    w = W.randn_bf16((n, k), W.SEED_MOE, "w", W.WEIGHTS, std=0.02, device=DEV)
    ref = None
    for t in (1, 64, 512):
        ids = list(range(1, t))
        ids.insert(t // 3, 0)
        a = W.rows_for_requests(ids, k, W.SEED_MOE, device=DEV)
        row = bi.bi_gemm(a, w, out_dtype=torch.float32)[t // 3].clone()
        if ref is None:
            ref = row
            assert_f32_close(row[None], O.gemm(f64(a[t // 3:t // 3 + 1]), f64(w)), "lm_head slice")
        assert_bitwise(row, ref, f"lm_head token 0 at T={t}")


def test_gemm_wide_tile_gives_the_same_bits():
    """A weight of at least 32768 rows runs the 128 x 256 tile (256 x 256 from
    512 rows on), a narrower one the 64 x 64 tile; all take every element's
    fp32 MFMA chain over k in the same order, so the tile changes no bit.  The same columns computed as one
    wide weight and as two narrow slices must agree bitwise (bf16 and fp32
    outputs, ragged m and n tails), and integer inputs must give the oracle
    rounded once on the wide path too."""
    k, n = 320, 32768 + 200
    w = W.randn_bf16((n, k), 11, "w", 1, std=0.05, device=DEV)
    for m in (1, 37, 300, 600):
        log_case(f"gemm wide tile m={m} n={n} k={k}")
        a = W.randn_bf16((m, k), 11, "x", m, device=DEV)
        cut = n // 2
        for dt in (torch.bfloat16, torch.float32):
            wide = bi.bi_gemm(a, w, out_dtype=dt)
            narrow = torch.cat([bi.bi_gemm(a, w[:cut], out_dtype=dt), bi.bi_gemm(a, w[cut:], out_dtype=dt)], dim=1)
            assert_bitwise(wide, narrow, f"wide vs narrow tile m={m} {dt}")
        ref = O.gemm(f64(a), f64(w[::97]))
        assert_bf16_close(bi.bi_gemm(a, w)[:, ::97], ref, f"wide tile parity m={m}")
        assert_f32_close(wide[:, ::97], ref, f"wide tile fp32 parity m={m}")
    ai, wi = _int_bf16((3, 256), 5), _int_bf16((33000, 256), 6)
    want = torch.from_numpy(O.f64_to_bf16_bits(O.gemm(f64(ai), f64(wi))).view(np.int16))
    assert torch.equal(bi.bi_gemm(ai.to(DEV), wi.to(DEV)).view(torch.int16).cpu(), want)


@pytest.mark.parametrize("n,k", [(12288 + 72, 4096), (4096, 12288), (6144, 4096)])
def test_gemm_large_m_rule_gives_the_same_bits(n, k):
    """Above 128 rows the tile comes from the round-count estimate (the
    Qwen3-8B step weights at M = 1024, 1100 and 2300, the up projection with a
    ragged n tail).  The whole product must equal, bit for bit, the same rows
    computed in slices of at most 512 rows, in bf16 and fp32."""
    w = W.randn_bf16((n, k), 12, "w", n, std=0.02, device=DEV)
    for m in (1024, 1100, 2300):
        log_case(f"gemm large-m rule m={m} n={n} k={k} tile={bi.gemm_tile(m, n, k)}")
        a = W.randn_bf16((m, k), 12, "x", m, device=DEV)
        for dt in (torch.bfloat16, torch.float32):
            whole = bi.bi_gemm(a, w, out_dtype=dt)
            sliced = torch.cat([bi.bi_gemm(a[r:r + 512], w, out_dtype=dt) for r in range(0, m, 512)])
            assert_bitwise(whole, sliced, f"large-m rule m={m} n={n} {dt}")
        ref = O.gemm(f64(a[::97]), f64(w[::89]))
        assert_bf16_close(bi.bi_gemm(a, w)[::97, ::89], ref, f"large-m rule parity m={m} n={n}")
        assert_f32_close(whole[::97, ::89], ref, f"large-m rule fp32 parity m={m} n={n}")


# Every tile the rule may pick above 128 rows, with the weight shapes searched
# for a product that reaches it (the rule depends on m, n, k and the device's
# compute units, so the test finds its shapes instead of fixing them).
LARGE_M_TILES = [(256, 256), (256, 192), (192, 256), (256, 160), (256, 128), (128, 256), (192, 128),
                 (128, 192), (128, 128), (64, 128), (64, 64)]
SEARCH_NK = [(n, k) for k in (4096, 512) for n in (1024, 2048, 4096, 6144, 12288)]


def _find_m(tile, limit=4400):
    for n, k in SEARCH_NK:
        for m in range(129, limit, 7):
            if bi.gemm_tile(m, n, k) == tile:
                return m, n, k
    return None


@pytest.mark.parametrize("tile", LARGE_M_TILES)
def test_gemm_every_large_m_tile_gives_the_same_bits(tile):
    """For each tile of the large-M rule, a product the rule runs on it must
    equal, bit for bit, the same rows computed in 128-row slices (which run the
    medium-M tiles), in bf16 and fp32, and sampled entries the oracle."""
    found = _find_m(tile)
    assert found is not None, f"no shape reaches tile {tile}"
    m, n, k = found
    log_case(f"gemm tile {tile}: m={m} n={n} k={k}")
    w = W.randn_bf16((n, k), 14, "w", n + k, std=0.02, device=DEV)
    a = W.randn_bf16((m, k), 14, "x", m, device=DEV)
    for dt in (torch.bfloat16, torch.float32):
        whole = bi.bi_gemm(a, w, out_dtype=dt)
        sliced = torch.cat([bi.bi_gemm(a[r:r + 128], w, out_dtype=dt) for r in range(0, m, 128)])
        assert_bitwise(whole, sliced, f"tile {tile} m={m} n={n} k={k} {dt}")
    ref = O.gemm(f64(a[::131]), f64(w[::113]))
    assert_f32_close(whole[::131, ::113], ref, f"tile {tile} fp32 parity")


def _rule_edges(n, k, lo=129, hi=4400, limit=4):
    """Consecutive m where the rule's tile changes."""
    out, prev = [], bi.gemm_tile(lo, n, k)
    for m in range(lo + 1, hi):
        t = bi.gemm_tile(m, n, k)
        if t != prev:
            out.append((m - 1, m, prev, t))
            if len(out) >= limit:
                break
        prev = t
    return out


@pytest.mark.parametrize("n,k", [(12288, 4096), (6144, 4096), (4096, 12288)])
def test_gemm_tile_rule_edges(n, k):
    """At the first rows counts where the large-M rule changes tile for the
    Qwen3-8B weights, m_lo and m_hi = m_lo + 1 run different tiles; the rows
    the two products share, and both products against the same rows in
    256-row slices, must agree bit for bit."""
    edges = _rule_edges(n, k)
    assert edges, f"the rule never changes tile for n={n} k={k}"
    w = W.randn_bf16((n, k), 13, "w", n, std=0.02, device=DEV)
    for m_lo, m_hi, t_lo, t_hi in edges:
        a = W.randn_bf16((m_hi, k), 13, "x", m_hi, device=DEV)
        log_case(f"gemm tile rule edge n={n} k={k} m={m_lo}/{m_hi}: {t_lo} -> {t_hi}")
        for dt in (torch.bfloat16, torch.float32):
            lo = bi.bi_gemm(a[:m_lo], w, out_dtype=dt)
            hi = bi.bi_gemm(a, w, out_dtype=dt)
            sliced = torch.cat([bi.bi_gemm(a[r:r + 256], w, out_dtype=dt) for r in range(0, m_hi, 256)])
            assert_bitwise(hi[:m_lo], lo, f"rows shared by m={m_lo} and m={m_hi} ({dt})")
            assert_bitwise(hi, sliced, f"m={m_hi} vs 256-row slices ({dt})")


@pytest.mark.parametrize("n,k", [(4096, 12288), (4097, 512), (6144, 4096), (8192, 512), (8200, 512),
                                 (12288, 4096), (16383, 512), (16384, 512)])
def test_gemm_small_m_tile_edges(n, k):
    """Up to 16 rows every weight narrower than the wide rule runs the 32 x 16
    tile (from 16384 weight rows, up to 32 rows, the 32 x 64 tile); up to 64
    rows a weight of at most 4096 rows runs the 16 x 64 tile and one of at most
    8192 rows the 32 x 64 tile; from 65 rows (or above 8192 weight rows) the
    larger tiles.  Rows shared by M = 1,
    16, 17, 64 and 65, and 16- and 32-row slices, must agree bit for bit, and
    integer inputs must give the oracle rounded once on the small-M paths."""
    w = W.randn_bf16((n, k), 14, "w", n, std=0.02, device=DEV)
    a = W.randn_bf16((65, k), 14, "x", k, device=DEV)
    log_case(f"gemm small-M tile edges n={n} k={k}")
    for dt in (torch.bfloat16, torch.float32):
        c65 = bi.bi_gemm(a, w, out_dtype=dt)
        for m in (64, 17, 16, 1):
            cm = bi.bi_gemm(a[:m].contiguous(), w, out_dtype=dt)
            assert_bitwise(c65[:m], cm, f"rows at M={m} vs M=65 ({dt})")
        for step in (16, 32):
            sl = torch.cat([bi.bi_gemm(a[r:r + step].contiguous(), w, out_dtype=dt) for r in range(0, 65, step)])
            assert_bitwise(c65, sl, f"M=65 vs {step}-row slices ({dt})")
    for m, rs in ((64, 16), (16, 5)):
        ref = O.gemm(f64(a[:m:rs]), f64(w[::37]))
        assert_bf16_close(bi.bi_gemm(a[:m].contiguous(), w)[::rs, ::37], ref, f"small-M parity n={n} M={m}")
    wi = _int_bf16((n, 256), 16)
    for rows in (7, 40):
        ai = _int_bf16((rows, 256), 15)
        want = torch.from_numpy(O.f64_to_bf16_bits(O.gemm(f64(ai), f64(wi))).view(np.int16))
        assert torch.equal(bi.bi_gemm(ai.to(DEV), wi.to(DEV)).view(torch.int16).cpu(), want)


@pytest.mark.parametrize("n", [4096, 4097, 6144, 12288])
def test_gemm_medium_m_tile_edges(n):
    """From 65 rows bi_gemm runs the 32 x 64 tile up to 128 rows for weights
    of at most 4096 rows, else the largest of the 128 x 128, 64 x 128 and
    64 x 64 tiles whose grid has at least 192 tiles (for N = 4096 the switches
    sit at M = 128/129, 256/257 and 640/641; for 4097 at 256/257 and 640/641;
    for 6144 at 128/129 and 384/385; for 12288 at 128/129).  Whole products at
    M on both sides of every switch must equal, row for row, the same rows
    computed as 64-row slices (the small-M tiles), bf16 and fp32, and integer
    inputs must give the oracle rounded once on the medium tiles (100 rows:
    the 32 x 64 tile at N = 4096; 300 rows: a medium tile)."""
    k = 512
    w = W.randn_bf16((n, k), 17, "w", n, std=0.05, device=DEV)
    a = W.randn_bf16((700, k), 17, "x", k, device=DEV)
    log_case(f"gemm medium-M tile edges n={n}")
    for dt in (torch.bfloat16, torch.float32):
        sl = torch.cat([bi.bi_gemm(a[r:r + 64].contiguous(), w, out_dtype=dt) for r in range(0, 700, 64)])
        for m in (65, 128, 129, 256, 257, 384, 385, 640, 641, 700):
            cm = bi.bi_gemm(a[:m].contiguous(), w, out_dtype=dt)
            assert_bitwise(cm, sl[:m], f"n={n} M={m} vs 64-row slices ({dt})")
    wi = _int_bf16((n, 256), 19)
    for rows in (100, 300):
        ai = _int_bf16((rows, 256), 18)
        want = torch.from_numpy(O.f64_to_bf16_bits(O.gemm(f64(ai), f64(wi))).view(np.int16))
        assert torch.equal(bi.bi_gemm(ai.to(DEV), wi.to(DEV)).view(torch.int16).cpu(), want)


def test_gemm_wide_tile_batch_invariance():
    # The full lm_head (4096 -> 151936, the wide tile): token 0's fp32 logits at
    # T in {1, 64, 512} and shuffled positions.
    k, n = 4096, 151936
    w = W.randn_bf16((n, k), W.SEED_MOE, "w", W.WEIGHTS, std=0.02, device=DEV)
    ref = None
    for t in (1, 64, 512):
        pos = (t * 7) // 9
        ids = list(range(1, t))
        ids.insert(pos, 0)
        a = W.rows_for_requests(ids, k, W.SEED_MOE, device=DEV)
        row = bi.bi_gemm(a, w, out_dtype=torch.float32)[pos].clone()
        if ref is None:
            ref = row
            assert_f32_close(row[None, ::61], O.gemm(f64(a[pos:pos + 1]), f64(w[::61])), "full lm_head")
        assert_bitwise(row, ref, f"full lm_head token 0 at T={t} slot={pos}")


def test_gemm_run_to_run():
    a = W.rows_for_requests(range(64), 4096, 2, device=DEV)
    w = W.randn_bf16((6144, 4096), 2, "w", 1, std=0.02, device=DEV)
    c0 = bi.bi_gemm(a, w)
    for _ in range(10):
        assert_bitwise(bi.bi_gemm(a, w), c0, "gemm repeat")


def test_gemm_errors():
    a = torch.ones((4, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bi.BiError) as e:
        bi.bi_gemm(a, a)
    assert e.value.status == bi.BI_ERR_UNSUPPORTED
    out = bi.bi_gemm(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV),
                     torch.ones((8, 64), dtype=torch.bfloat16, device=DEV))
    assert out.shape == (0, 8)
