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
    """The Qwen3-8B step weights at M = 1024, 1100 and 2300 (the up projection
    with a ragged n tail): the whole product must equal, bit for bit, the same
    rows computed in slices of at most 512 rows, in bf16 and fp32."""
    w = W.randn_bf16((n, k), 12, "w", n, std=0.02, device=DEV)
    for m in (1024, 1100, 2300):
        log_case(f"gemm large-m rule m={m} n={n} k={k} config={bi.gemm_config(m, n, k)}")
        a = W.randn_bf16((m, k), 12, "x", m, device=DEV)
        for dt in (torch.bfloat16, torch.float32):
            whole = bi.bi_gemm(a, w, out_dtype=dt)
            sliced = torch.cat([bi.bi_gemm(a[r:r + 512], w, out_dtype=dt) for r in range(0, m, 512)])
            assert_bitwise(whole, sliced, f"large-m rule m={m} n={n} {dt}")
        ref = O.gemm(f64(a[::97]), f64(w[::89]))
        assert_bf16_close(bi.bi_gemm(a, w)[::97, ::89], ref, f"large-m rule parity m={m} n={n}")
        assert_f32_close(whole[::97, ::89], ref, f"large-m rule fp32 parity m={m} n={n}")


# Every configuration of the estimate-based rule (tile n, tile m, wavefronts n,
# m, stages, K per stage, workgroups per CU, non-temporal weight loads).  The rule depends on m, n, k and
# the device's compute units, so the tests search for a product that reaches
# each configuration instead of fixing its shape.
_BASE_CONFIGS = [(256, 256, 2, 4, 2, 64, 1), (256, 192, 2, 4, 2, 64, 1), (192, 256, 2, 4, 2, 64, 1),
                 (256, 160, 2, 2, 3, 64, 1), (256, 128, 2, 4, 3, 64, 1), (128, 256, 2, 4, 3, 64, 1),
                 (192, 128, 2, 2, 4, 64, 1), (128, 192, 2, 2, 4, 64, 1), (96, 192, 2, 2, 4, 64, 1),
                 (128, 128, 2, 2, 4, 64, 1), (96, 128, 2, 2, 5, 64, 1), (64, 128, 2, 2, 3, 64, 2),
                 (96, 64, 2, 2, 4, 64, 2), (64, 64, 2, 2, 5, 64, 2), (64, 64, 2, 2, 4, 128, 1),
                 (32, 64, 2, 2, 6, 64, 2), (32, 64, 2, 2, 4, 128, 1), (32, 32, 2, 2, 8, 128, 1),
                 (16, 64, 1, 4, 4, 128, 2), (16, 64, 1, 4, 8, 128, 1), (32, 16, 2, 1, 6, 128, 2)]
# The last field: weight loads non-temporal (tiles of at most 64 rows holding all m rows).
RULE_CONFIGS = [c + (0,) for c in _BASE_CONFIGS] + [c + (1,) for c in _BASE_CONFIGS if c[1] <= 64]
SEARCH_NK = [(n, k) for k in (4096, 512, 12288) for n in (4096, 6144, 12288, 24576, 1024, 2048, 8192)]
SEARCH_M = list(range(1, 257)) + list(range(257, 4400, 7))


def _find_shape(cfg):
    for n, k in SEARCH_NK:
        for m in SEARCH_M:
            if bi.gemm_config(m, n, k) == cfg:
                return m, n, k
    return None


def _reference_rows(a, w, dt, m):
    """The rows of a w^T computed under another configuration than m rows get:
    64-row slices above 64 rows, else the head of a 300-row batch."""
    if m > 64:
        return torch.cat([bi.bi_gemm(a[r:r + 64], w, out_dtype=dt) for r in range(0, m, 64)])
    extra = W.randn_bf16((300 - m, a.shape[1]), 15, "x", 300, device=DEV)
    return bi.bi_gemm(torch.cat([a, extra]), w, out_dtype=dt)[:m]


@pytest.mark.parametrize("cfg", RULE_CONFIGS, ids=lambda c: "x".join(map(str, c)))
def test_gemm_every_configuration_gives_the_same_bits(cfg):
    """For each configuration the rule can pick, a product the rule runs on it
    must equal, bit for bit, the same rows computed under another
    configuration, in bf16 and fp32, and sampled entries the oracle."""
    found = _find_shape(cfg)
    if found is None:
        pytest.skip(f"the rule picks {cfg} for none of the searched shapes")
    m, n, k = found
    w = W.randn_bf16((n, k), 14, "w", n + k, std=0.02, device=DEV)
    a = W.randn_bf16((m, k), 14, "x", m, device=DEV)
    other = bi.gemm_config(64 if m > 64 else 300, n, k)
    log_case(f"gemm config {cfg}: m={m} n={n} k={k}, reference rows on {other}")
    assert other != cfg
    for dt in (torch.bfloat16, torch.float32):
        whole = bi.bi_gemm(a, w, out_dtype=dt)
        assert_bitwise(whole, _reference_rows(a, w, dt, m), f"config {cfg} m={m} n={n} k={k} {dt}")
    ref = O.gemm(f64(a[::131]), f64(w[::113]))
    assert_f32_close(whole[::131, ::113], ref, f"config {cfg} fp32 parity")


def _rule_edges(n, k, lo=1, hi=4400):
    """Consecutive m where the rule's configuration changes."""
    out, prev = [], bi.gemm_config(lo, n, k)
    for m in range(lo + 1, hi + 1):
        c = bi.gemm_config(m, n, k)
        if c != prev:
            out.append((m - 1, m, prev, c))
        prev = c
    return out


@pytest.mark.parametrize("n,k", [(12288, 4096), (6144, 4096), (4096, 12288), (4096, 4096), (24576, 4096),
                                 (4097, 512), (8200, 512)])
def test_gemm_tile_rule_edges(n, k):
    """At every rows count up to 4400 where the rule changes configuration for
    these weights (the Qwen3-8B projections and two ragged ones), m_lo and
    m_hi = m_lo + 1 run different kernels; the rows the two products share,
    and the larger product against the same rows in slices (64 rows up to
    1100, else 256), must agree bit for bit."""
    edges = _rule_edges(n, k)
    assert edges, f"the rule never changes configuration for n={n} k={k}"
    w = W.randn_bf16((n, k), 13, "w", n, std=0.02, device=DEV)
    a_all = W.randn_bf16((edges[-1][1], k), 13, "x", 4400, device=DEV)
    for m_lo, m_hi, c_lo, c_hi in edges:
        a = a_all[:m_hi]
        log_case(f"gemm tile rule edge n={n} k={k} m={m_lo}/{m_hi}: {c_lo} -> {c_hi}")
        step = 64 if m_hi <= 1100 else 256
        for dt in (torch.bfloat16, torch.float32):
            lo = bi.bi_gemm(a[:m_lo], w, out_dtype=dt)
            hi = bi.bi_gemm(a, w, out_dtype=dt)
            assert_bitwise(hi[:m_lo], lo, f"rows shared by m={m_lo} and m={m_hi} ({dt})")
            if m_hi > 64:
                sliced = torch.cat([bi.bi_gemm(a[r:r + step], w, out_dtype=dt) for r in range(0, m_hi, step)])
                assert_bitwise(hi, sliced, f"m={m_hi} vs {step}-row slices ({dt})")
            del lo, hi


@pytest.mark.parametrize("k", [192, 160, 4096])
def test_gemm_exact_zero_sign_is_batch_invariant(k):
    """Rows of A that are all -0.0 against positive weights make every product
    -0.0.  Tiles whose last K stage is only partly inside K run extra MFMA
    steps on zeros; the rule keeps every candidate on the same side of that
    (at k = 192 no tile with 128-wide stages is used), so the sign of such an
    exact zero must be the same at every M (compared bitwise against the rows
    alone)."""
    n = 4096
    w = (W.randn_bf16((n, k), 16, "w", k, std=0.02, device=DEV).float().abs() + 0.01).to(torch.bfloat16)
    a = W.randn_bf16((600, k), 16, "x", k, device=DEV)
    for r in (0, 37, 599):
        a[r] = -0.0
    log_case(f"gemm -0 rows k={k}")
    for dt in (torch.bfloat16, torch.float32):
        single = {r: bi.bi_gemm(a[r:r + 1], w, out_dtype=dt) for r in (0, 37, 599)}
        for m in (1, 8, 38, 64, 65, 128, 129, 256, 300, 600):
            c = bi.bi_gemm(a[:m], w, out_dtype=dt)
            for r in (0, 37, 599):
                if r < m:
                    assert_bitwise(c[r:r + 1], single[r], f"-0 row {r} at M={m} k={k} ({dt})")


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
