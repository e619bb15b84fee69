"""bi_moe_ffn on the GPU: parity with the fp64 oracle (small shapes in full,
the Qwen3-235B-A22B expert shape on sampled tokens), the pages' property (a
token's output bits do not depend on the other tokens of the batch, their
number, or the token's position), skewed and degenerate routing, errors."""
import numpy as np
import pytest
import torch

import workloads as W
from _helpers import O, assert_bf16_close, assert_bitwise, bi, ensure_lib, f64, log_case

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
    """Token 0's output bits at T = 1, 8, 64, 512, at shuffled positions."""
    w_up, w_down = full_weights
    ref = None
    for T, slot in ((1, 0), (8, 0), (8, 5), (64, 37), (512, 300)):
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
