"""Pins for the fp64 oracle: closed forms, exact brute force on tiny inputs,
invariants and the pages' worked example.  CPU only.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, index or axis, a transposed operand, sum instead of mean, a missing
scale) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 coding

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x3F81, 0x0000, 0x8000, 0x4049],
                    dtype=np.uint16)
    v = O.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == math.inf and v[3] == -math.inf
    assert v[4] == 2.0 ** -133                      # smallest subnormal
    assert v[5] == 1.0 + 2.0 ** -7
    assert v[6] == 0.0 and math.copysign(1.0, v[7]) == -1.0
    assert v[8] == 3.140625


def test_bf16_round_trip_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f64(bits)
    finite = np.isfinite(v)
    back = O.f64_to_bf16_bits(v[finite])
    assert np.array_equal(back, bits[finite])


def test_bf16_rounding_ties_to_even_and_direct():
    one = 1.0
    cases = {
        one + 2.0 ** -8: 0x3F80,                    # tie, even neighbour is 1.0
        one + 3 * 2.0 ** -8: 0x3F82,                # tie, even neighbour is 1 + 2^-6
        one + 2.0 ** -8 + 2.0 ** -40: 0x3F81,       # just above the tie (fp32 would lose this bit)
        -(one + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        3.0e38 * 2: 0x7F80,                         # overflow
        2.0 ** -134: 0x0000,                        # half the smallest subnormal: tie to even (zero)
        3 * 2.0 ** -134: 0x0002,                    # 1.5 quanta: tie to even (2 quanta)
    }
    for x, want in cases.items():
        assert int(O.f64_to_bf16_bits(np.array([x]))[0]) == want, x


def test_bf16_rounding_matches_independent_fp32_path():
    # For float32-representable inputs a float32 -> bf16 RNE (torch) must agree.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(x32.astype(np.float64))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_row_of_ones():
    for H in (1, 7, 512, 4096):
        eps = 1e-6
        y = O.rmsnorm(np.ones((1, H)), np.ones(H), eps)
        assert np.allclose(y, 1.0 / math.sqrt(1.0 + eps), rtol=0, atol=1e-15)


def test_rmsnorm_constant_row_and_gain():
    H, c, eps = 64, -3.5, 1e-3
    g = np.linspace(0.5, 2.0, H)
    y = O.rmsnorm(np.full((2, H), c), g, eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps) * g, rtol=1e-15, atol=0)


def test_rmsnorm_zero_row_and_one_hot():
    H, eps = 32, 1e-6
    assert np.all(O.rmsnorm(np.zeros((1, H)), np.ones(H), eps) == 0.0)
    a, k = 5.0, 11
    g = np.arange(1, H + 1, dtype=np.float64)
    x = np.zeros((1, H))
    x[0, k] = a
    y = O.rmsnorm(x, g, eps)
    want = np.zeros(H)
    want[k] = a / math.sqrt(a * a / H + eps) * g[k]
    assert np.allclose(y[0], want, rtol=1e-15, atol=0)


def test_rmsnorm_mean_square_closed_form_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 96))
    ms = np.mean(x * x, axis=1)
    eps = 0.25
    y = O.rmsnorm(x, np.ones(96), eps)
    # mean(y^2) = ms / (ms + eps): catches sum-vs-mean, eps outside the root, H-1.
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13, atol=0)
    y0 = O.rmsnorm(x, np.ones(96), 0.0)
    assert np.allclose(O.rmsnorm(37.0 * x, np.ones(96), 0.0), y0, rtol=1e-13, atol=0)


def test_rmsnorm_exact_sum_of_squares_brute_force():
    # Dyadic inputs: the mean square is an exact rational; eps = 0 and a mean
    # square that is a perfect square make the whole result exact.
    x = np.array([[3.0, -4.0, 0.0, 0.0], [1.0, 1.0, 1.0, -1.0]])   # ms = 25/4 and 1
    for r in range(2):
        ms = sum(Fraction(v) ** 2 for v in x[r]) / 4
        root = {Fraction(25, 4): Fraction(5, 2), Fraction(1): Fraction(1)}[ms]
        want = [float(Fraction(v) / root) for v in x[r]]
        assert list(O.rmsnorm(x[r:r + 1], np.ones(4), 0.0)[0]) == want


# ---------------------------------------------------------------- GEMM

def test_gemm_integer_brute_force_exact():
    rng = np.random.default_rng(2)
    M, N, K = 5, 7, 13
    a = rng.integers(-4, 5, (M, K))
    w = rng.integers(-4, 5, (N, K))
    want = [[sum(int(a[m, k]) * int(w[n, k]) for k in range(K)) for n in range(N)] for m in range(M)]
    got = O.gemm(a.astype(np.float64), w.astype(np.float64))
    assert got.shape == (M, N)
    assert got.tolist() == [[float(v) for v in row] for row in want]


def test_gemm_identity_ones_and_selector():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((4, 6))
    assert np.array_equal(O.gemm(a, np.eye(6)), a)
    assert np.all(O.gemm(np.ones((3, 9)), np.ones((2, 9))) == 9.0)
    w = rng.standard_normal((5, 6))
    sel = np.zeros((2, 6))
    sel[0, 4] = 1.0
    sel[1, 1] = 1.0
    c = O.gemm(sel, w)                      # row m picks column i_m of W: C[m, n] = W[n, i_m]
    assert np.array_equal(c[0], w[:, 4]) and np.array_equal(c[1], w[:, 1])


# ---------------------------------------------------------------- attention

def test_chunk_decomposition_matches_pages_example():
    with open(os.path.join(GOLDEN, "chunk_example.json")) as f:
        g = json.load(f)
    assert O.KV_CHUNK == g["chunk"]
    assert O.kv_chunks(g["length"]) == g["chunks"]


def test_chunk_decomposition_prefix_stable():
    # Finished chunks never change as the cache grows (chunks anchored at 0).
    for L in range(0, 2000, 37):
        for L2 in (L + 1, L + 255, L + 700):
            a, b = O.kv_chunks(L), O.kv_chunks(L2)
            assert sum(a) == L and all(c == 256 for c in a[:-1])
            full = L // 256
            assert b[:full] == a[:full]


def test_attention_single_token_exact():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal(64), rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    o, lse = O.attention_row(q, k, v, 0.125)
    assert np.array_equal(o, v[0])
    assert lse == pytest.approx(0.125 * float(q @ k[0]), abs=1e-15)


def test_attention_uniform_cases():
    rng = np.random.default_rng(5)
    L, D = 300, 16
    k, v = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    o, lse = O.attention_row(np.zeros(D), k, v, 0.3)          # q = 0: uniform weights
    assert np.allclose(o, v.mean(axis=0), rtol=0, atol=1e-14)
    assert lse == pytest.approx(math.log(L), abs=1e-13)
    kk = np.tile(rng.standard_normal(D), (L, 1))                # identical keys: uniform
    o2, _ = O.attention_row(rng.standard_normal(D), kk, v, 0.3)
    assert np.allclose(o2, v.mean(axis=0), rtol=0, atol=1e-14)
    vv = np.tile(rng.standard_normal(D), (L, 1))                # identical values: o = v
    o3, _ = O.attention_row(rng.standard_normal(D), k, vv, 0.3)
    assert np.allclose(o3, vv[0], rtol=0, atol=1e-14)


def test_attention_two_keys_logistic_closed_form():
    rng = np.random.default_rng(6)
    D, scale = 8, 0.7
    q, k, v = rng.standard_normal(D), rng.standard_normal((2, D)), rng.standard_normal((2, D))
    s0, s1 = scale * float(q @ k[0]), scale * float(q @ k[1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))                        # logistic weight of key 0
    o, lse = O.attention_row(q, k, v, scale)
    assert np.allclose(o, w0 * v[0] + (1.0 - w0) * v[1], rtol=0, atol=1e-14)
    assert lse == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), abs=1e-14)


def test_attention_spike_closed_form():
    # One key with score a, the other L-1 with score b: weights are closed-form.
    L, D = 50, 4
    q = np.array([1.0, 0, 0, 0])
    k = np.zeros((L, D))
    k[7, 0] = 3.0
    v = np.zeros((L, D))
    v[:, 1] = 1.0
    v[7] = [0, 0, 5.0, 0]
    scale = 0.5
    ea, eb = math.exp(scale * 3.0), 1.0
    den = ea + (L - 1) * eb
    o, lse = O.attention_row(q, k, v, scale)
    assert np.allclose(o, [0, (L - 1) * eb / den, 5.0 * ea / den, 0], rtol=0, atol=1e-15)
    assert lse == pytest.approx(math.log(den), abs=1e-14)


def test_decode_gqa_head_mapping():
    B, Hq, Hkv, D, L = 2, 8, 2, 4, 5
    rng = np.random.default_rng(8)
    q = rng.standard_normal((B, Hq, D))
    ks = [rng.standard_normal((L, Hkv, D)) for _ in range(B)]
    vs = []
    for b in range(B):
        v = np.zeros((L, Hkv, D))
        for g in range(Hkv):
            v[:, g, :] = 10 * b + g + 1                        # constant per (request, kv head)
        vs.append(v)
    out, _ = O.decode_attention(q, ks, vs, 0.5)
    for b in range(B):
        for h in range(Hq):
            assert np.allclose(out[b, h], 10 * b + h // (Hq // Hkv) + 1, atol=1e-14)


def test_prefill_causal_mask_and_decode_equivalence():
    rng = np.random.default_rng(9)
    P, n, Hq, Hkv, D = 20, 6, 4, 2, 8
    k = rng.standard_normal((P + n, Hkv, D))
    v = rng.standard_normal((P + n, Hkv, D))
    q = rng.standard_normal((n, Hq, D))
    out, lse = O.prefill_attention(q, k, v, P, 0.35)
    # Keys after a query's position must not matter: poison every key past
    # position P + i and hand the oracle the whole poisoned cache and chunk.
    # Rows 0..i see only clean keys and must not move; a mask that lets row i
    # see one key too many picks up the poison.
    for i in range(n):
        k2, v2 = k.copy(), v.copy()
        k2[P + i + 1:] = 1e3
        v2[P + i + 1:] = -1e3
        o2, l2 = O.prefill_attention(q, k2, v2, P, 0.35)
        assert np.allclose(o2[:i + 1], out[:i + 1], atol=1e-13) and np.allclose(l2[:i + 1], lse[:i + 1], atol=1e-13)
        if i + 1 < n:
            assert not np.allclose(o2[i + 1], out[i + 1], atol=1e-3), "the poison reaches the next row"
        od, ld = O.decode_attention(q[i:i + 1], [k[:P + i + 1]], [v[:P + i + 1]], 0.35)
        assert np.allclose(od[0], out[i], atol=1e-13) and np.allclose(ld[0], lse[i], atol=1e-13)
    # The first chunk query with P = 0 sees exactly one key: o = v0.
    o0, _ = O.prefill_attention(q[:1], k[:1], v[:1], 0, 0.35)
    for h in range(Hq):
        assert np.array_equal(o0[0, h], v[0, h // 2])


@pytest.mark.parametrize("L", [1, 255, 256, 257, 1000, 4096])
def test_fixed_size_split_merge_identity(L):
    rng = np.random.default_rng(L)
    D = 32
    q = rng.standard_normal(D) * 2
    k, v = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    o1, l1 = O.attention_row(q, k, v, 0.4)
    o2, l2 = O.chunked_attention_row(q, k, v, 0.4)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)
    assert abs(l1 - l2) < 1e-12


def test_merge_single_partial_and_order_free_in_exact_arithmetic():
    m, l, acc = 1.5, 3.0, np.array([3.0, -6.0])
    o, lse = O.merge_partials([(m, l, acc)])
    assert np.array_equal(o, acc / l) and lse == pytest.approx(m + math.log(l), abs=1e-15)
    parts = [(0.0, 1.0, np.array([1.0, 0.0])), (math.log(3.0), 1.0, np.array([0.0, 1.0]))]
    o2, lse2 = O.merge_partials(parts)              # weights 1 : 3
    assert np.allclose(o2, [0.25, 0.75], atol=1e-15)
    assert lse2 == pytest.approx(math.log(4.0), abs=1e-15)


# ---------------------------------------------------------------- log_softmax

def test_log_softmax_closed_forms():
    V = 151936
    lp = O.log_softmax(np.full((1, V), 3.25))
    assert np.allclose(lp, -math.log(V), atol=1e-12)
    z = np.array([[2.0, -1.0]])
    lp2 = O.log_softmax(z)
    assert lp2[0, 0] == pytest.approx(-math.log1p(math.exp(-3.0)), abs=1e-15)
    assert lp2[0, 1] == pytest.approx(-math.log1p(math.exp(3.0)), abs=1e-15)
    rng = np.random.default_rng(10)
    zz = rng.standard_normal((3, 1000)) * 5
    lpz = O.log_softmax(zz)
    assert np.allclose(np.exp(lpz).sum(axis=1), 1.0, atol=1e-13)
    assert np.allclose(O.log_softmax(zz + 123.0), lpz, atol=1e-12)
    assert np.all(np.argmax(lpz, axis=1) == np.argmax(zz, axis=1))


# ---------------------------------------------------------------- MoE support

def test_silu_closed_form():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([math.log(3.0)]))[0] == pytest.approx(0.75 * math.log(3.0), abs=1e-15)
    assert O.silu(np.array([-math.log(3.0)]))[0] == pytest.approx(-0.25 * math.log(3.0), abs=1e-15)


def test_moe_routing_and_weighting():
    rng = np.random.default_rng(11)
    T, H, E, k = 3, 4, 5, 2
    x = rng.standard_normal((T, H))
    w_up = [np.eye(H) for _ in range(E)]
    w_down = [(e + 1) * np.eye(H) for e in range(E)]             # expert e scales by e + 1
    experts = np.array([[0, 3], [4, 1], [2, 2]])
    weights = np.array([[0.25, 0.75], [0.5, 0.5], [0.1, 0.2]])
    y = O.moe_ffn(x, experts, weights, w_up, w_down)
    sx = x / (1.0 + np.exp(-x))
    for t in range(T):
        scale = sum(weights[t, s] * (experts[t, s] + 1) for s in range(k))
        assert np.allclose(y[t], scale * sx[t], atol=1e-14)


# ---------------------------------------------------------------- decoder layer (composition)

def test_moe_route_closed_forms():
    # Equal logits: the tie-break takes the lowest expert indices, weights 1/k.
    x = np.ones((2, 4))
    experts, weights, logits = O.moe_route(x, np.zeros((16, 4)), 8)
    assert experts.tolist() == [list(range(8))] * 2
    assert np.array_equal(weights, np.full((2, 8), 1 / 8))
    assert np.array_equal(logits, np.zeros((2, 16)))
    # One-hot token and gate rows c_e e_0: logits are c_e; the top 3 of
    # c = [0, 5, -1, 5, 2] are experts 1, 3 (tie, lower index first), 4.
    c = np.array([0.0, 5.0, -1.0, 5.0, 2.0])
    w_gate = np.zeros((5, 3))
    w_gate[:, 0] = c
    experts, weights, _ = O.moe_route(np.array([[1.0, 0.0, 0.0]]), w_gate, 3)
    assert experts[0].tolist() == [1, 3, 4]
    z = np.exp(np.array([5.0, 5.0, 2.0]) - 5.0)
    assert np.allclose(weights[0], z / z.sum(), rtol=0, atol=1e-15)
    # Two experts: the weights are the logistic function of the logit gap.
    experts, weights, _ = O.moe_route(np.array([[2.0]]), np.array([[0.25], [1.0]]), 2)
    assert experts[0].tolist() == [1, 0]
    assert abs(weights[0, 0] - 1 / (1 + math.exp(-1.5))) < 1e-15


def test_moe_route_brute_force():
    # Small integer inputs: exact logits; the chosen set is the k-subset of
    # largest logit sum with the lexicographically smallest indices among ties,
    # listed by (-logit, index); found here by enumerating every k-subset.
    import itertools
    rng = np.random.default_rng(11)
    for _ in range(30):
        E, k, H = int(rng.integers(3, 9)), int(rng.integers(1, 4)), 3
        x = rng.integers(-2, 3, (1, H)).astype(float)
        w = rng.integers(-2, 3, (E, H)).astype(float)
        lg = (w @ x[0])
        best = None
        for sub in itertools.combinations(range(E), k):
            key = (-sum(lg[list(sub)]), sorted(sub))
            if best is None or key < best[0]:
                best = (key, sub)
        want = sorted(best[1], key=lambda e: (-lg[e], e))
        experts, weights, logits = O.moe_route(x, w, k)
        assert np.array_equal(logits[0], lg)
        assert experts[0].tolist() == want, (lg, experts[0], want)
        assert abs(weights[0].sum() - 1.0) < 1e-12 and np.all(np.diff(weights[0]) <= 0)


def test_silu_mul_halves_and_closed_form():
    # g = ln 3 -> silu = 0.75 ln 3; the first half gates, the second multiplies
    gu = np.array([[math.log(3.0), 0.0, 2.0, 5.0]])
    out = O.silu_mul(gu)
    assert out.shape == (1, 2)
    assert out[0, 0] == pytest.approx(0.75 * math.log(3.0) * 2.0, abs=1e-14)
    assert out[0, 1] == 0.0                                    # silu(0) = 0, whatever u is
    # silu(x) - silu(-x) = x (sigma(x) + sigma(-x) = 1): the gate is the first half
    x = np.array([0.3, -1.7, 4.0])
    a = O.silu_mul(np.concatenate([x, np.ones(3)])[None])[0]
    b = O.silu_mul(np.concatenate([-x, np.ones(3)])[None])[0]
    assert np.allclose(a - b, x, atol=1e-14)


def _tiny_layer(rng, H=16, hq=2, hkv=1, d=8, F=16):
    r = lambda *s: O.round_bf16(rng.standard_normal(s) * 0.3)
    return dict(g1=O.round_bf16(1.0 + 0.1 * rng.standard_normal(H)), g2=O.round_bf16(1.0 + 0.1 * rng.standard_normal(H)),
                w_qkv=r((hq + 2 * hkv) * d, H), w_o=r(H, hq * d), w_gu=r(2 * F, H), w_down=r(H, F))


def test_decoder_layer_residual_path():
    """With W_o = W_down = 0 both branches add exact zeros: y is x itself, and
    k, v are the rounded projection of the rounded rmsnorm of x."""
    rng = np.random.default_rng(5)
    H, hq, hkv, d = 16, 2, 1, 8
    w = _tiny_layer(rng)
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    x = O.round_bf16(rng.standard_normal((3, H)))
    kp, vp = O.round_bf16(rng.standard_normal((5, hkv, d))), O.round_bf16(rng.standard_normal((5, hkv, d)))
    y, k, v = O.decoder_layer(x, kp, vp, w, hq, hkv, d, 1e-6, 0.35)
    assert np.array_equal(y, x)
    qkv = O.round_bf16(O.round_bf16(O.rmsnorm(x, w["g1"], 1e-6)) @ w["w_qkv"].T)
    assert np.array_equal(k.reshape(3, -1), qkv[:, hq * d:(hq + hkv) * d])
    assert np.array_equal(v.reshape(3, -1), qkv[:, (hq + hkv) * d:])


def test_decoder_layer_wiring_closed_forms():
    """Single-token sequence (attention = its own v), W_qkv's v block and W_o the
    identity: r = round(x + h).  Then gate = I, up = 2 I, W_down = I:
    y = round(r + round(silu(h2) * 2 h2)) - which a swapped gate/up
    (silu(2 h2) * h2) or a residual taken from h instead of x would miss."""
    rng = np.random.default_rng(6)
    H = 8
    hq = hkv = 1
    d = H
    eye = np.eye(H)
    w = dict(g1=O.round_bf16(1.0 + 0.1 * rng.standard_normal(H)), g2=O.round_bf16(1.0 + 0.1 * rng.standard_normal(H)),
             w_qkv=np.concatenate([rng.standard_normal((H, H)), rng.standard_normal((H, H)), eye]),
             w_o=eye, w_gu=np.concatenate([eye, 2.0 * eye]), w_down=eye)
    w["w_qkv"] = O.round_bf16(w["w_qkv"])
    x = O.round_bf16(rng.standard_normal((1, H)))
    empty = np.zeros((0, hkv, d))
    y, _, v = O.decoder_layer(x, empty, empty, w, hq, hkv, d, 1e-6, 0.5)
    h = O.round_bf16(O.rmsnorm(x, w["g1"], 1e-6))
    assert np.array_equal(v.reshape(1, H), h)                   # v = h (identity block)
    r = O.round_bf16(x + h)                                    # attention over one key returns v exactly
    h2 = O.round_bf16(O.rmsnorm(r, w["g2"], 1e-6))
    m = O.round_bf16(O.silu(h2) * O.round_bf16(2.0 * h2))
    assert np.array_equal(y, O.round_bf16(r + m))
    swapped = O.round_bf16(O.silu(O.round_bf16(2.0 * h2)) * h2)
    assert not np.array_equal(m, swapped)
