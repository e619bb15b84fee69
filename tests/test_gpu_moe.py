"""bi_moe_ffn on the GPU: parity with the fp64 oracle (small shapes in full,
the Qwen3-235B-A22B expert shape on sampled tokens), the pages' property (a
token's output bits do not depend on the other tokens of the batch, their
number, or the token's position), skewed and degenerate routing, errors."""
import numpy as np
import pytest
import torch

import workloads as W
from _helpers import O, assert_bf16_close, assert_bitwise, assert_f32_close, bi, ensure_lib, f64, log_case

pytestmark = pytest.mark.gpu
DEV = "cuda"
E_FULL, K_FULL, H_FULL, F_FULL = 128, 8, 4096, 1536


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _oracle(x, experts, weights, w_up, w_down, tokens):
    """Oracle rows for `tokens`; slots with an out-of-range expert id are dropped."""
    E = w_up.shape[0]
    out = []
    for t in tokens:
        ex, wt = experts[t].numpy().copy(), weights[t].numpy().astype(np.float64)
        keep = (ex >= 0) & (ex < E)
        ex, wt = np.where(keep, ex, 0), np.where(keep, wt, 0.0)
        used = sorted(set(int(e) for e in ex))
        ups = {e: f64(w_up[e]) for e in used}
        downs = {e: f64(w_down[e]) for e in used}
        out.append(O.moe_ffn(f64(x[t:t + 1]), ex[None, :], wt[None, :],
                             [ups.get(e) for e in range(max(used) + 1)],
                             [downs.get(e) for e in range(max(used) + 1)])[0])
    return np.stack(out)


@pytest.mark.parametrize("T,E,k,H,F", [(37, 16, 4, 256, 192), (1, 8, 2, 64, 32), (130, 5, 3, 96, 224)])
def test_moe_parity_small(T, E, k, H, F):
    log_case(f"moe parity T={T} E={E} k={k} H={H} F={F}")
    x = W.rows_for_requests(range(T), H, W.SEED_MOE)
    experts, weights = W.moe_routing(range(T), E, k, W.SEED_MOE)
    w_up, w_down = W.moe_weights(E, H, F, W.SEED_MOE, std_up=H ** -0.5, std_down=F ** -0.5)
    y = bi.bi_moe_ffn(x.to(DEV), experts.to(DEV), weights.to(DEV), w_up.to(DEV), w_down.to(DEV))
    torch.cuda.synchronize()
    ref = _oracle(x, experts, weights, w_up, w_down, range(T))
    assert_bf16_close(y.cpu(), ref, "moe small")


@pytest.fixture(scope="module")
def full_weights():
    return W.moe_weights(E_FULL, H_FULL, F_FULL, W.SEED_MOE, device=DEV)


def _tokens(ids):
    x = W.rows_for_requests(ids, H_FULL, W.SEED_MOE)
    experts, weights = W.moe_routing(ids, E_FULL, K_FULL, W.SEED_MOE)
    return x, experts, weights


def test_moe_parity_full_shape_sampled(full_weights):
    w_up, w_down = full_weights
    T = 64
    log_case(f"moe full shape T={T}, oracle on sampled tokens")
    x, experts, weights = _tokens(range(T))
    y = bi.bi_moe_ffn(x.to(DEV), experts.to(DEV), weights.to(DEV), w_up, w_down).cpu()
    for t in (0, 29, 63):
        ex = experts[t].tolist()
        ups = {e: f64(w_up[e]) for e in ex}
        downs = {e: f64(w_down[e]) for e in ex}
        ref = O.moe_ffn(f64(x[t:t + 1]), np.arange(K_FULL)[None, :], weights[t:t + 1].numpy().astype(np.float64),
                        [ups[e] for e in ex], [downs[e] for e in ex])
        assert_bf16_close(y[t:t + 1], ref, f"moe full shape token {t}")


def test_moe_batch_invariance(full_weights):
    """Token 0's output bits at T = 1, 8, 64, 511, 512, 513, 2048, at shuffled
    positions (above 32 rows per expert, T = 513 with 128 experts and top 8,
    the grouped GEMMs switch from the 64 x 64 to the 128 x 256 tile)."""
    w_up, w_down = full_weights
    ref = None
    for T, slot in ((1, 0), (8, 0), (8, 5), (64, 37), (511, 200), (512, 300), (513, 400), (2048, 1500),
                    (2048, 2047)):
        log_case(f"moe invariance T={T} slot={slot}")
        others = list(range(1, T))
        ids = others[:slot] + [0] + others[slot:]
        x, experts, weights = _tokens(ids)
        y = bi.bi_moe_ffn(x.to(DEV), experts.to(DEV), weights.to(DEV), w_up, w_down)[slot].cpu()
        if ref is None:
            ref = y
        else:
            assert_bitwise(y, ref, f"token 0 at T={T} slot={slot}")


def test_moe_skewed_routing_invariance(full_weights):
    """Every token routed to the same 8 experts (each expert gets all T rows)."""
    w_up, w_down = full_weights
    ref = None
    for T in (1, 3, 200):
        log_case(f"moe skewed T={T}")
        x, _, weights = _tokens(range(T))
        experts = torch.arange(K_FULL, dtype=torch.int32).repeat(T, 1)
        y = bi.bi_moe_ffn(x.to(DEV), experts.to(DEV), weights.to(DEV), w_up, w_down).cpu()
        if ref is None:
            ref = y[0]
            ups = {e: f64(w_up[e]) for e in range(K_FULL)}
            downs = {e: f64(w_down[e]) for e in range(K_FULL)}
            want = O.moe_ffn(f64(x[:1]), experts[:1].numpy(), weights[:1].numpy().astype(np.float64),
                             [ups[e] for e in range(K_FULL)], [downs[e] for e in range(K_FULL)])
            assert_bf16_close(y[:1], want, "skewed token 0")
        else:
            assert_bitwise(y[0], ref, f"skewed token 0 at T={T}")


def test_moe_dropped_slots_and_empty():
    T, E, k, H, F = 9, 6, 3, 64, 64
    x = W.rows_for_requests(range(T), H, W.SEED_MOE)
    experts, weights = W.moe_routing(range(T), E, k, W.SEED_MOE)
    experts[2, 1] = -1
    experts[5, 0] = E        # out of range: dropped
    experts[7, :] = -1       # every slot dropped: y = 0
    w_up, w_down = W.moe_weights(E, H, F, W.SEED_MOE, std_up=H ** -0.5, std_down=F ** -0.5)
    y = bi.bi_moe_ffn(x.to(DEV), experts.to(DEV), weights.to(DEV), w_up.to(DEV), w_down.to(DEV)).cpu()
    ref = _oracle(x, experts, weights, w_up, w_down, [t for t in range(T) if t != 7])
    assert_bf16_close(torch.cat([y[:7], y[8:]]), ref, "dropped slots")
    assert torch.equal(y[7].view(torch.int16), torch.zeros(H, dtype=torch.int16))
    # no tokens: a no-op
    out = torch.full((0, H), 1.0, dtype=torch.bfloat16, device=DEV)
    bi.bi_moe_ffn(x[:0].to(DEV), experts[:0].to(DEV), weights[:0].to(DEV), w_up.to(DEV), w_down.to(DEV), out=out)


def test_moe_errors():
    T, E, k, H, F = 4, 4, 2, 64, 64
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    wt = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    w_up = torch.zeros((E, F, H), dtype=torch.bfloat16, device=DEV)
    w_down = torch.zeros((E, H, F), dtype=torch.bfloat16, device=DEV)
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(bi.BiError) as e:
        bi.bi_moe_ffn(x, ids, wt, w_up, w_down, workspace=small)
    assert e.value.status == bi.BI_ERR_WORKSPACE
    bad_h = torch.zeros((T, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bi.BiError) as e:
        bi.bi_moe_ffn(bad_h, ids, wt, torch.zeros((E, F, 48), dtype=torch.bfloat16, device=DEV),
                      torch.zeros((E, 48, F), dtype=torch.bfloat16, device=DEV))
    assert e.value.status == bi.BI_ERR_UNSUPPORTED


# ---------------------------------------------------------------- the router (bi_moe_route)

def _gate(E=E_FULL, H=H_FULL):
    return W.randn_bf16((E, H), W.SEED_MOE, "gate", W.WEIGHTS, std=0.02)


def _order(lg, k):
    """Top-k of every row of lg in the router's order: larger first, lower index on ties."""
    return np.array([sorted(range(lg.shape[1]), key=lambda e: (-lg[t, e], e))[:k] for t in range(lg.shape[0])])


@pytest.mark.parametrize("T", [1, 37, 300])
def test_moe_route_parity(T):
    """Logits against the oracle (fp32 absolute); the choice - an integer decided
    by floating point - exactly equal to the order of the library's own fp32
    logits, and equal to the oracle's where its top k + 1 logits are clearly
    apart; the weights against the oracle's softmax of its logits of the chosen
    experts."""
    log_case(f"moe route parity T={T}")
    x, wg = W.rows_for_requests(range(T), H_FULL, W.SEED_MOE), _gate()
    ids, wts, logits = bi.bi_moe_route(x.to(DEV), wg.to(DEV), K_FULL)
    ref_ids, ref_w, ref_lg = O.moe_route(f64(x), f64(wg), K_FULL)
    assert_f32_close(logits, ref_lg, f"router logits T={T}")
    ids_np, lg = ids.cpu().numpy(), logits.cpu().double().numpy()
    assert np.array_equal(ids_np, _order(lg, K_FULL)), "choice = order of the library's fp32 logits"
    top = -np.sort(-ref_lg, axis=1)[:, :K_FULL + 1]
    clear = np.all(-np.diff(top, axis=1) > 1e-3, axis=1)
    assert clear.sum() >= max(1, T // 2)
    assert np.array_equal(ids_np[clear], ref_ids[clear]), "choice = oracle's where the logits are apart"
    for t in range(T):
        z = ref_lg[t, ids_np[t]]
        p = np.exp(z - z.max())
        assert np.max(np.abs(wts[t].cpu().double().numpy() - p / p.sum())) <= 1e-3
    assert np.allclose(wts.cpu().double().numpy().sum(axis=1), 1.0, atol=1e-6)


def test_moe_route_ties_and_closed_forms():
    x = W.rows_for_requests(range(5), 512, W.SEED_MOE).to(DEV)
    # A zero gate: every logit is 0, so experts 0..7 by the tie-break, weights exactly 1/8.
    ids, wts, lg = bi.bi_moe_route(x, torch.zeros((128, 512), dtype=torch.bfloat16, device=DEV), 8)
    assert torch.equal(ids.cpu(), torch.arange(8, dtype=torch.int32).repeat(5, 1))
    assert torch.equal(wts.cpu(), torch.full((5, 8), 0.125))
    assert torch.equal(lg.cpu(), torch.zeros((5, 128)))
    # Expert e + 64 repeats expert e's gate row: bitwise equal logits, so every
    # chosen expert e is followed by e + 64, with the same weight.
    g = W.randn_bf16((64, 512), W.SEED_MOE, "gate", 77, std=0.05).to(DEV)
    ids, wts, lg = bi.bi_moe_route(x, torch.cat([g, g]).contiguous(), 8)
    assert_bitwise(lg[:, :64], lg[:, 64:], "duplicated gate rows")
    ids = ids.cpu()
    assert torch.equal(ids[:, 0::2] + 64, ids[:, 1::2]), ids
    assert torch.all(ids[:, 0::2] < 64)
    assert_bitwise(wts[:, 0::2], wts[:, 1::2], "tied weights")
    # Many experts (the 16-per-lane instance): E = 300 and 1024, top 16.
    for E in (300, 1024):
        ge = W.randn_bf16((E, 512), W.SEED_MOE, "gate", 1000 + E, std=0.05).to(DEV)
        ids, wts, lg = bi.bi_moe_route(x, ge, 16)
        assert np.array_equal(ids.cpu().numpy(), _order(lg.cpu().double().numpy(), 16)), f"E={E}"
        assert np.allclose(wts.cpu().double().numpy().sum(axis=1), 1.0, atol=1e-6)
    # E = 5, top_k = 5: every expert, in logit order.
    ids, wts, lg = bi.bi_moe_route(x, g[:5].contiguous(), 5)
    assert np.array_equal(ids.cpu().numpy(), _order(lg.cpu().double().numpy(), 5))


def test_moe_route_batch_invariance():
    """Token 0's logits, choice and weights: bitwise the same at T = 1, 64, 512,
    2048 and shuffled positions."""
    wg = _gate().to(DEV)
    ref = None
    for T, slot in ((1, 0), (64, 37), (512, 300), (512, 0), (2048, 777)):
        log_case(f"moe route invariance T={T} slot={slot}")
        others = list(range(1, T))
        ids_ = others[:slot] + [0] + others[slot:]
        x = W.rows_for_requests(ids_, H_FULL, W.SEED_MOE, device=DEV)
        ids, wts, lg = bi.bi_moe_route(x, wg, K_FULL)
        got = (ids[slot].clone(), wts[slot].clone(), lg[slot].clone())
        if ref is None:
            ref = got
        for a, b, what in zip(got, ref, ("ids", "weights", "logits")):
            assert_bitwise(a, b, f"token 0 {what} at T={T} slot={slot}")


def test_moe_layer_routed_invariance_and_parity(full_weights):
    """The whole routed layer (bi_moe_route then bi_moe_ffn): token 0's output
    bitwise the same at T = 1, 64, 512, 2048; and against the oracle's routed
    layer on tokens whose routing is clear."""
    w_up, w_down = full_weights
    wg = _gate().to(DEV)
    ref = None
    for T, slot in ((1, 0), (64, 10), (512, 411), (2048, 1234)):
        log_case(f"routed moe layer T={T} slot={slot}")
        others = list(range(1, T))
        ids_ = others[:slot] + [0] + others[slot:]
        x = W.rows_for_requests(ids_, H_FULL, W.SEED_MOE, device=DEV)
        ids, wts, _ = bi.bi_moe_route(x, wg, K_FULL)
        y = bi.bi_moe_ffn(x, ids, wts, w_up, w_down)
        if ref is None:
            ref = y[slot].clone()
            ex, rw, rl = O.moe_route(f64(x[:1]), f64(wg), K_FULL)
            ex = ex[0].tolist()
            assert ids[0].cpu().tolist() == ex
            ups = [f64(w_up[e]) for e in ex]
            downs = [f64(w_down[e]) for e in ex]
            yr = O.moe_ffn(f64(x[:1]), np.arange(K_FULL)[None, :], rw, ups, downs)
            assert_bf16_close(y[:1], yr, "routed layer vs oracle")
        assert_bitwise(y[slot], ref, f"routed layer token 0 at T={T} slot={slot}")
