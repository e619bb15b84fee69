"""A whole pre-norm decoder layer (invariant_bi_rmsnorm_02_amd.layer) on the GPU:
parity with the oracle's layer at a reduced shape, and at the Qwen3-8B shape a
token's layer output - and the K/V it appends - bitwise the same whatever it
is batched with, and whether its chunk is prefilled in one call or decoded one
token at a time."""
import numpy as np
import pytest
import torch

import workloads as W
from _helpers import O, assert_bf16_close, assert_bitwise, bi, ensure_lib, f64, log_case, row_rel_err
from invariant_bi_rmsnorm_02_amd.layer import DecoderLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")
EPS = 1e-6
SEED = 61


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _layer(H, hq, hkv, d, F, seed=SEED):
    w = lambda n, k, i: W.randn_bf16((n, k), seed, "w", i, std=0.02, device=DEV)
    g = lambda i: W.randn_bf16((H,), seed, "gamma", i, std=0.1, mean=1.0, device=DEV)
    return DecoderLayer(w((hq + 2 * hkv) * d, H, 1), w(H, hq * d, 2), w(2 * F, H, 3), w(H, F, 4), g(5), g(6),
                        hq, hkv, d, EPS)


def _np_weights(layer):
    return dict(g1=f64(layer.g1), g2=f64(layer.g2), w_qkv=f64(layer.w_qkv), w_o=f64(layer.w_o),
                w_gu=f64(layer.w_gu), w_down=f64(layer.w_down))


class Caches:
    """Sequences whose caches hold `prefix[s]` earlier tokens (random K/V) and
    have room for `new[s]` more; unused slots are NaN."""

    def __init__(self, prefix, new, hkv, d, seed, perm_index=0):
        self.prefix, self.new = list(prefix), list(new)
        total = [p + n for p, n in zip(prefix, new)]
        self.pb = W.allocate_pages(total, seed, 16, 3, perm_index)
        self.kc, self.vc = bi.alloc_kv_cache(self.pb.num_pages, hkv, d, 16, fill=NAN)
        self.kv = [W.request_kv(900 + s, p, hkv, d, seed, device=DEV) for s, p in enumerate(prefix)]
        self.bt = self.pb.block_table.to(DEV)
        starts = np.cumsum([0] + total[:-1]).tolist()
        self.slots = [self.pb.slot_mapping[st:st + t].to(DEV) for st, t in zip(starts, total)]
        for s, p in enumerate(prefix):
            if p:
                bi.bi_kv_append(self.kv[s][0], self.kv[s][1], self.slots[s][:p], self.kc, self.vc)


def _tokens(n, H, seed, tag):
    return W.randn_bf16((n, H), seed, "x", tag, device=DEV)


@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 4096), (257, 1032), (0, 64)])
def test_add_parity(rows, cols):
    """bf16(x + y): the fp32 sum of two bf16 values rounds to the same bf16 as
    the exact sum (exact when the exponents differ by at most 16, else far
    from a rounding midpoint), so the result is bit-exact."""
    log_case(f"add rows={rows} cols={cols}")
    x = W.randn_bf16((rows, cols), SEED, "x", 7, device=DEV)
    y = W.randn_bf16((rows, cols), SEED, "x", 8, std=3e-3, device=DEV)
    if rows > 2:
        y[1] = -x[1]                      # exact cancellation to +0
        y[2, :8] = x[2, :8] * 2.0 ** -20  # far-apart exponents
    out = bi.bi_add(x, y)
    torch.cuda.synchronize()
    want = O.f64_to_bf16_bits(O.round_bf16(f64(x) + f64(y))).view(np.int16)
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), want.reshape(rows, cols))


def test_add_strided_and_in_place():
    x = W.randn_bf16((40, 3 * 512), SEED, "x", 9, device=DEV)
    a, b = x[:, :512], x[:, 1024:]
    want = bi.bi_add(a.contiguous(), b.contiguous())
    assert_bitwise(bi.bi_add(a, b), want, "strided add")
    c = a.clone()
    bi.bi_add(c, b, out=c)
    assert_bitwise(c, want, "in-place add")


@pytest.mark.parametrize("rows,f", [(1, 8), (5, 12288), (129, 1544), (0, 16)])
def test_silu_mul_parity(rows, f):
    """silu(g) * u in fp32 with one rounding: within one bf16 ulp of the
    correctly rounded value, and equal to it for nearly every element."""
    log_case(f"silu_mul rows={rows} f={f}")
    gu = W.randn_bf16((rows, 2 * f), SEED, "x", 10, std=2.0, device=DEV)
    out = bi.bi_silu_mul(gu)
    torch.cuda.synchronize()
    ref = O.round_bf16(O.silu_mul(f64(gu)))
    got = f64(out)
    if rows == 0:
        assert got.shape == (0, f)
        return
    ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(got - ref) <= ulp), "silu_mul off by more than one bf16 ulp"
    assert np.mean(got == ref) >= 0.99, f"silu_mul: only {np.mean(got == ref):.4f} exactly rounded"


def test_silu_mul_closed_forms():
    """silu(0) = 0, silu(g) -> g for large g and -> -0 for very negative g;
    u = 1 returns silu(g) itself."""
    g = torch.tensor([0.0, 40.0, -200.0, 1.0, -1.0, 2.0, 3.0, -3.0], dtype=torch.bfloat16, device=DEV)
    gu = torch.cat([g, torch.ones(8, dtype=torch.bfloat16, device=DEV)]).view(1, 16)
    got = f64(bi.bi_silu_mul(gu))[0]
    assert got[0] == 0.0 and got[1] == 40.0 and got[2] == 0.0
    ref = O.round_bf16(O.silu_mul(f64(gu)))[0]
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7)


def test_pointwise_validation():
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError):
        bi.bi_add(x, x)                          # cols not a multiple of 8
    with pytest.raises(RuntimeError):
        bi.bi_silu_mul(torch.zeros((4, 24), dtype=torch.bfloat16, device=DEV))   # f = 12
    with pytest.raises(RuntimeError):
        bi.bi_add(torch.zeros((4, 16), dtype=torch.bfloat16, device=DEV)[:, 1:9],
                  torch.zeros((4, 8), dtype=torch.bfloat16, device=DEV))        # misaligned base


def _padded(rows, cols, pad, seed, tag, std=1.0):
    """A [rows, cols] bf16 view whose rows are `cols + pad` elements apart."""
    buf = W.randn_bf16((rows, cols + pad), seed, "x", tag, std=std, device=DEV)
    return buf[:, :cols]


# (M, N, K): the decode and mixed-batch shapes of the O and down projections
# (tiles from 16 x 64 to 256 x 160 under the rule), and small shapes with a ragged
# last n-group (N % 4 != 0).
GEMM_ADD_SHAPES = [(1, 4096, 4096), (16, 4096, 12288), (17, 4096, 4096), (64, 4096, 12288), (65, 4096, 4096),
                   (128, 4096, 12288), (300, 4096, 4096), (700, 4096, 4096), (2300, 4096, 12288),
                   (5, 100, 64), (37, 38, 96), (130, 202, 128)]


@pytest.mark.parametrize("m,n,k", GEMM_ADD_SHAPES)
def test_gemm_add_equals_unfused(m, n, k):
    """bi_gemm_add is bit for bit bi_gemm (bf16) followed by bi_add: into a new
    tensor, in place (y = x) and with padded row strides."""
    log_case(f"gemm_add m={m} n={n} k={k}")
    a = W.randn_bf16((m, k), SEED, "x", 20, device=DEV)
    w = W.randn_bf16((n, k), SEED, "w", 21, std=0.02, device=DEV)
    pad = 8 - n % 8 if n % 8 else 8
    x = _padded(m, n, pad, SEED, 22)
    c = torch.empty((m, n + pad), dtype=torch.bfloat16, device=DEV)[:, :n]
    bi.bi_gemm(a, w, out=c)
    want = torch.empty_like(c)
    if n % 8 == 0:
        bi.bi_add(x, c, out=want)
    else:   # bi_add takes widths in multiples of 8: run it on the padded rows
        xp, cp = x.as_strided((m, n + pad), x.stride()), c.as_strided((m, n + pad), c.stride())
        cp[:, n:] = 0
        wp = torch.empty((m, n + pad), dtype=torch.bfloat16, device=DEV)
        bi.bi_add(xp, cp, out=wp)
        want = wp[:, :n]
    got = torch.empty((m, n + pad), dtype=torch.bfloat16, device=DEV)[:, :n]
    bi.bi_gemm_add(a, w, x, out=got)
    assert_bitwise(got, want, f"gemm_add {m}x{n}x{k}")
    if n % 8 == 0:
        assert_bitwise(bi.bi_gemm_add(a, w, x), want, f"gemm_add, new output {m}x{n}x{k}")
    y = x.as_strided((m, n + pad), x.stride()).clone()[:, :n]
    bi.bi_gemm_add(a, w, y, out=y)
    assert_bitwise(y, want, f"gemm_add in place {m}x{n}x{k}")


# (M, f, K): the gate/up projection of the decode and mixed-batch layers on
# every tile of the rule, and small shapes (f odd: a last (gate, up) pair alone).
GEMM_SILU_SHAPES = [(1, 12288, 4096), (16, 12288, 4096), (32, 12288, 4096), (33, 12288, 4096),
                    (64, 12288, 4096), (65, 12288, 4096), (256, 12288, 4096), (1100, 12288, 4096),
                    (3, 8, 64), (20, 25, 96), (70, 203, 128)]


@pytest.mark.parametrize("m,f,k", GEMM_SILU_SHAPES)
def test_gemm_silu_mul_equals_unfused(m, f, k):
    """bi_gemm_silu_mul on the row-interleaved weight is bit for bit bi_gemm on
    the [gate; up] weight followed by bi_silu_mul."""
    log_case(f"gemm_silu_mul m={m} f={f} k={k}")
    a = W.randn_bf16((m, k), SEED, "x", 23, device=DEV)
    w = W.randn_bf16((2 * f, k), SEED, "w", 24, std=0.05, device=DEV)
    w_il = bi.interleave_gate_up(w)
    assert_bitwise(w_il[0::2], w[:f], "interleaved gate rows")
    assert_bitwise(w_il[1::2], w[f:], "interleaved up rows")
    gu = bi.bi_gemm(a, w)
    fp = (f + 7) // 8 * 8       # bi_silu_mul takes f in multiples of 8: pad with zero columns
    gp = torch.zeros((m, 2 * fp), dtype=torch.bfloat16, device=DEV)
    gp[:, :f], gp[:, fp:fp + f] = gu[:, :f], gu[:, f:]
    want = bi.bi_silu_mul(gp)[:, :f]
    if f % 8 == 0:
        assert_bitwise(bi.bi_gemm_silu_mul(a, w_il), want, f"gemm_silu_mul {m}x{f}x{k}")
    out = torch.full((m, fp + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    bi.bi_gemm_silu_mul(a, w_il, out=out[:, :f])
    assert_bitwise(out[:, :f], want, f"gemm_silu_mul strided out {m}x{f}x{k}")
    assert bool(torch.isnan(out[:, f:].float()).all()), "gemm_silu_mul wrote past f"


def test_fused_gemm_oracle_parity():
    """The fused calls against the oracle's definitions (bf16 product rounded,
    then the elementwise step in fp64 and one rounding): within one bf16 ulp of
    the oracle on the elementwise step, given the GEMM's bf16 output."""
    m, n, k = 37, 96, 256
    a = W.randn_bf16((m, k), SEED, "x", 25, device=DEV)
    w = W.randn_bf16((n, k), SEED, "w", 26, std=0.05, device=DEV)
    x = W.randn_bf16((m, n), SEED, "x", 27, device=DEV)
    y = f64(bi.bi_gemm_add(a, w, x))
    c = f64(bi.bi_gemm(a, w))
    assert_bf16_close(bi.bi_gemm(a, w), O.gemm(f64(a), f64(w)), "gemm_add's product")
    assert np.array_equal(y, O.round_bf16(f64(x) + c)), "gemm_add: x + bf16(product) not correctly rounded"
    f = n // 2
    wg = W.randn_bf16((2 * f, k), SEED, "w", 28, std=0.05, device=DEV)
    h = f64(bi.bi_gemm_silu_mul(a, bi.interleave_gate_up(wg)))
    gu = f64(bi.bi_gemm(a, wg))
    ref = O.round_bf16(O.silu_mul(gu))
    ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(h - ref) <= ulp), "gemm_silu_mul off by more than one bf16 ulp"


def test_fused_gemm_validation():
    a = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((16, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        bi.bi_gemm_add(a, w, torch.zeros((4, 8), dtype=torch.bfloat16, device=DEV))     # x not [m, n]
    with pytest.raises(RuntimeError):
        bi.bi_gemm_add(a, w, torch.zeros((4, 20), dtype=torch.bfloat16, device=DEV)[:, 2:18])  # misaligned x
    with pytest.raises(ValueError):
        bi.bi_gemm_silu_mul(a, torch.zeros((15, 64), dtype=torch.bfloat16, device=DEV))  # odd row count
    with pytest.raises(RuntimeError):
        bi.bi_gemm_silu_mul(a, w, out=torch.zeros((4, 12), dtype=torch.bfloat16, device=DEV)[:, :8])  # ldo


U = 2.0 ** -8      # unit roundoff of bf16 (8 significant bits, round to nearest)


def _check_steps(tr, x, k_prefix, v_prefix, npw, hq, hkv, d, scale, what):
    """Every library call of the layer against the oracle's step applied to
    the call's own GPU inputs, at the per-kernel tolerance (bf16 outputs: max
    relative error <= 1e-2 against the row scale), and the two residual adds
    bit-exact (the correctly rounded sum of the same two bf16 inputs)."""
    T = x.shape[0]
    h, qkv, a = f64(tr["h"]), f64(tr["qkv"]), f64(tr["attn"]).reshape(T, hq * d)
    c, r, h2, gu, m, dn = (f64(tr[n]) for n in ("c", "r", "h2", "gu", "m", "d"))
    assert_bf16_close(tr["h"], O.rmsnorm(x, npw["g1"], EPS), f"{what}: rmsnorm 1")
    assert_bf16_close(tr["qkv"], O.gemm(h, npw["w_qkv"]), f"{what}: qkv projection")
    q = qkv[:, :hq * d].reshape(T, hq, d)
    K = np.concatenate([k_prefix, qkv[:, hq * d:(hq + hkv) * d].reshape(T, hkv, d)])
    V = np.concatenate([v_prefix, qkv[:, (hq + hkv) * d:].reshape(T, hkv, d)])
    ra, _ = O.prefill_attention(q, K, V, k_prefix.shape[0], scale)
    assert_bf16_close(tr["attn"], ra, f"{what}: attention")
    assert_bf16_close(tr["c"], O.gemm(a, npw["w_o"]), f"{what}: o projection")
    assert np.array_equal(r, O.round_bf16(x + c)), f"{what}: residual add 1 not bit-exact"
    assert_bf16_close(tr["h2"], O.rmsnorm(r, npw["g2"], EPS), f"{what}: rmsnorm 2")
    assert_bf16_close(tr["gu"], O.gemm(h2, npw["w_gu"]), f"{what}: gate/up projection")
    assert_bf16_close(tr["m"], O.silu_mul(gu), f"{what}: silu * up")
    assert_bf16_close(tr["d"], O.gemm(m, npw["w_down"]), f"{what}: down projection")
    return r, c, dn


def _check_end_to_end(y, x, tr_r, tr_c, tr_d, steps, what):
    """The layer output against the oracle's layer run from the same x.

    Both sides end with two correctly rounded adds on the residual stream,
    r = RN(x + c) and y = RN(r + d), over the same x; they differ only in the
    branch outputs c (o projection) and d (down projection).  With
    |RN(s) - s| <= U |s|, element by element:
        |y_g - y_o| <= |c_g - c_o| + |d_g - d_o|
                       + U (|x + c_g| + |x + c_o| + |r_g + d_g| + |r_o + d_o|).
    The last term is the two outputs' own roundings: two faithful evaluations
    may land on neighbouring bf16 values at each add, so the layer output can
    differ by up to two ulps (4U |y| ~ 1.6e-2 |y|) with no error on either side,
    more than the 1e-2 a single kernel meets.  The branch outputs themselves,
    run end to end from x, stay within 1e-2 of the oracle's in norm."""
    yg, co, do, ro = f64(y), steps["c"], steps["d"], steps["r"]
    yo = steps["y"]
    bound = (np.abs(tr_c - co) + np.abs(tr_d - do)
             + U * (np.abs(x + tr_c) + np.abs(x + co) + np.abs(tr_r + tr_d) + np.abs(ro + do)))
    err = np.abs(yg - yo)
    assert np.all(err <= bound * (1 + 1e-12)), \
        f"{what}: layer output off its rounding bound at {np.unravel_index(np.argmax(err - bound), err.shape)}"
    for name, g, o in (("o projection", tr_c, co), ("down projection", tr_d, do), ("layer output", yg, yo)):
        nrel = float(np.linalg.norm(g - o) / np.linalg.norm(o))
        assert nrel <= 1e-2, f"{what}: {name} norm-wise relative error {nrel:.2e} > 1e-2"
    print(f"[layer] {what}: max elementwise rel err {row_rel_err(yg, yo):.3e}, "
          f"norm-wise {np.linalg.norm(yg - yo) / np.linalg.norm(yo):.2e}", flush=True)


def _oracle_layer(x, kp, vp, npw, hq, hkv, d, scale):
    steps = {}
    y, _, _ = O.decoder_layer(x, kp, vp, npw, hq, hkv, d, EPS, scale, steps=steps)
    steps["y"] = y
    return steps


SMALL = dict(H=1024, hq=8, hkv=2, d=128, F=2048)
QWEN = dict(H=4096, hq=32, hkv=8, d=128, F=12288)


@pytest.mark.parametrize("shape", ["small", "qwen3_8b"])
def test_layer_parity(shape):
    """The decoder layer at a reduced shape and at the Qwen3-8B shape (hidden
    4096, 32/8 heads, MLP 12288): decode of three sequences (caches of 0, 299
    and 699 tokens before the new one) and a chunked prefill of two sequences
    (40 and 100 new tokens after 0 and 260 cached).  Every step against the
    oracle at the per-kernel tolerance on its own inputs, the output against
    the oracle's layer under the rounding-propagation bound."""
    dims = SMALL if shape == "small" else QWEN
    H, hq, hkv, d = dims["H"], dims["hq"], dims["hkv"], dims["d"]
    layer = _layer(**dims)
    npw = _np_weights(layer)
    log_case(f"layer parity {shape}: decode")
    prefix = [0, 299, 699]
    c = Caches(prefix, [1, 1, 1], hkv, d, SEED)
    x = _tokens(3, H, SEED, 1)
    lens = torch.tensor([p + 1 for p in prefix], dtype=torch.int32, device=DEV)
    slots = torch.stack([c.slots[s][p] for s, p in enumerate(prefix)])
    tr = {}
    y = layer.decode(x, c.kc, c.vc, c.bt, lens, slots, 700, trace=tr)
    assert_bitwise(layer.decode(x, c.kc, c.vc, c.bt, lens, slots, 700), y, f"{shape} decode: fused vs traced")
    torch.cuda.synchronize()
    for s, p in enumerate(prefix):
        rows = slice(s, s + 1)
        sub = {k: v[rows] for k, v in tr.items()}
        xs, kp, vp = f64(x[rows]), f64(c.kv[s][0]), f64(c.kv[s][1])
        r, cg, dg = _check_steps(sub, xs, kp, vp, npw, hq, hkv, d, layer.scale, f"{shape} decode seq {s}")
        st = _oracle_layer(xs, kp, vp, npw, hq, hkv, d, layer.scale)
        _check_end_to_end(y[rows], xs, r, cg, dg, st, f"{shape} decode seq {s} (cache {p})")
    log_case(f"layer parity {shape}: prefill")
    prefix, new = [0, 260], [40, 100]
    c = Caches(prefix, new, hkv, d, SEED, perm_index=1)
    x = _tokens(sum(new), H, SEED, 2)
    q_start = torch.tensor([0, new[0], sum(new)], dtype=torch.int32, device=DEV)
    ctx = torch.tensor(prefix, dtype=torch.int32, device=DEV)
    slots = torch.cat([c.slots[s][p:p + n] for s, (p, n) in enumerate(zip(prefix, new))])
    tr = {}
    y = layer.prefill(x, c.kc, c.vc, c.bt, q_start, ctx, slots, max(new), trace=tr)
    assert_bitwise(layer.prefill(x, c.kc, c.vc, c.bt, q_start, ctx, slots, max(new)), y,
                   f"{shape} prefill: fused vs traced")
    torch.cuda.synchronize()
    for s, (p, n) in enumerate(zip(prefix, new)):
        rows = slice(int(q_start[s]), int(q_start[s + 1]))
        sub = {k: v[rows] for k, v in tr.items()}
        xs, kp, vp = f64(x[rows]), f64(c.kv[s][0]), f64(c.kv[s][1])
        r, cg, dg = _check_steps(sub, xs, kp, vp, npw, hq, hkv, d, layer.scale, f"{shape} prefill seq {s}")
        st = _oracle_layer(xs, kp, vp, npw, hq, hkv, d, layer.scale)
        _check_end_to_end(y[rows], xs, r, cg, dg, st, f"{shape} prefill seq {s}")




def test_layer_batch_invariance():
    """Request 0 (700 cached tokens) decodes its next token alone, among 8 and
    among 63 others of random lengths; its output row and the cache page its
    new K/V lands in are bitwise the same every time."""
    layer = _layer(**QWEN)
    x0 = _tokens(1, QWEN["H"], SEED, 3)
    ref = None
    for B, perm in ((1, 0), (9, 1), (64, 2)):
        log_case(f"layer batch invariance B={B}")
        prefix = [700] + [W.rand_int(1, 3000, SEED, "len", 50 + i) for i in range(B - 1)]
        c = Caches(prefix, [1] * B, QWEN["hkv"], QWEN["d"], SEED, perm_index=perm)
        x = torch.cat([x0, _tokens(B - 1, QWEN["H"], SEED, 100 + B)]) if B > 1 else x0
        lens = torch.tensor([p + 1 for p in prefix], dtype=torch.int32, device=DEV)
        slots = torch.stack([c.slots[s][p] for s, p in enumerate(prefix)])
        y = layer.decode(x, c.kc, c.vc, c.bt, lens, slots, max(prefix) + 1)
        assert bool(torch.isfinite(y).all()), f"non-finite layer output at B={B}"
        page = int(c.pb.block_table[0, 700 // 16])
        got = (y[0].clone(), c.kc[page].clone(), c.vc[page].clone())
        if ref is None:
            ref = got
            continue
        assert_bitwise(got[0], ref[0], f"layer output of request 0 at B={B}")
        assert_bitwise(got[1], ref[1], f"K page holding request 0's new token at B={B}")
        assert_bitwise(got[2], ref[2], f"V page holding request 0's new token at B={B}")


def test_layer_prefill_equals_decode():
    """A 40-token chunk after 300 cached tokens: prefilled in one call, or
    decoded one token at a time, gives bitwise the same output rows and
    leaves bitwise the same cache."""
    layer = _layer(**QWEN)
    P, n = 300, 40
    x = _tokens(n, QWEN["H"], SEED, 4)
    a = Caches([P], [n], QWEN["hkv"], QWEN["d"], SEED)
    b = Caches([P], [n], QWEN["hkv"], QWEN["d"], SEED)
    log_case("layer prefill vs decode")
    yp = layer.prefill(x, a.kc, a.vc, a.bt, torch.tensor([0, n], dtype=torch.int32, device=DEV),
                       torch.tensor([P], dtype=torch.int32, device=DEV), a.slots[0][P:P + n], n)
    assert bool(torch.isfinite(yp).all()), "non-finite prefill layer output"
    for i in range(n):
        yd = layer.decode(x[i:i + 1], b.kc, b.vc, b.bt, torch.tensor([P + i + 1], dtype=torch.int32, device=DEV),
                          b.slots[0][P + i:P + i + 1], P + n)
        assert_bitwise(yd[0], yp[i], f"token {i}: decode vs prefill")
    assert_bitwise(a.kc, b.kc, "K cache after prefill vs after decoding")
    assert_bitwise(a.vc, b.vc, "V cache after prefill vs after decoding")
