"""The Qwen3-235B-A22B-shaped layer as one path on the GPU: decode attention
(64 q / 4 kv heads, head_dim 128, paged caches of 1..4096 tokens) -> RMSNorm
-> router (128 experts, top 8) -> expert FFNs (4096 -> 1536 -> 4096) ->
residual -> RMSNorm -> lm_head 4096 -> 151936 with the fused log_softmax, and
the greedy token.  A tracked request's logprobs, greedy token and its
logprob must be bitwise the same whatever batch it is decoded in (T = 1, 64,
512, 2048 tokens per step, other requests drawn at random, the tracked one at
random slots) - the property the pages check with sampler/trainer logprobs -
and every step of the path must agree with the oracle applied to that step's
own inputs."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import (O, assert_bf16_close, assert_bitwise, assert_f32_close, bi, ensure_lib, f64, log_case)
from invariant_bi_rmsnorm_02_amd.layer import LMHead, MoEDecoderLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"
S = W.SEED_MOE
H, HQ, HKV, D, E, K, F, V = 4096, 64, 4, 128, 128, 8, 1536, 151936
POOL = 2048 + 64          # requests that can be drawn into a batch
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


@pytest.fixture(scope="module")
def model():
    w = lambda n, k, i: W.randn_bf16((n, k), S, "w", W.WEIGHTS + i, std=0.02, device=DEV)
    g = lambda i: W.randn_bf16((H,), S, "gamma", W.WEIGHTS + i, std=0.1, mean=1.0, device=DEV)
    w_up, w_down = W.moe_weights(E, H, F, S, device=DEV)
    layer = MoEDecoderLayer(w((HQ + 2 * HKV) * D, H, 301), w(H, HQ * D, 302),
                            W.randn_bf16((E, H), S, "gate", W.WEIGHTS, std=0.02, device=DEV), w_up, w_down,
                            g(303), g(304), HQ, HKV, D, K, EPS)
    head = LMHead(g(305), w(V, H, 306), EPS)
    return layer, head


@pytest.fixture(scope="module")
def pool():
    """POOL requests, each with L ~ U[1, 4096] cached tokens (seeded K/V) and
    room for one more, in one NaN-poisoned paged cache."""
    lens = W.decode_lengths(range(POOL), S, 1, 4096)
    pb = W.allocate_pages([L + 1 for L in lens], S, perm_index=7)
    kc, vc = bi.alloc_kv_cache(pb.num_pages, HKV, D, 16, fill=float("nan"))
    starts = np.cumsum([0] + [L + 1 for L in lens[:-1]]).tolist()
    kv = {}
    for r, L in enumerate(lens):
        k, v = W.request_kv(r, L, HKV, D, S, device=DEV)
        bi.bi_kv_append(k, v, pb.slot_mapping[starts[r]:starts[r] + L].to(DEV), kc, vc)
        if r == 0:
            kv[r] = (k, v)
    new_slot = torch.tensor([int(pb.slot_mapping[st + L]) for st, L in zip(starts, lens)], dtype=torch.int32)
    x = W.rows_for_requests(range(POOL), H, S, device=DEV)
    return dict(lens=lens, bt=pb.block_table.to(DEV), kc=kc, vc=vc, new_slot=new_slot.to(DEV), x=x, kv0=kv[0])


def _step(model, pool, ids, trace=None):
    layer, head = model
    idx = torch.tensor(ids, dtype=torch.long, device=DEV)
    lens = torch.tensor([pool["lens"][i] + 1 for i in ids], dtype=torch.int32, device=DEV)
    y = layer.decode(pool["x"][idx].contiguous(), pool["kc"], pool["vc"], pool["bt"][idx].contiguous(), lens,
                     pool["new_slot"][idx].contiguous(), 4097, trace=trace)
    lp = head.logprobs(y, trace=trace)
    tok, tlp = head.greedy(y)
    return y, lp, tok, tlp


def _compositions():
    rng = np.random.default_rng(55)
    out = []
    for T, slot in ((1, 0), (64, 17), (512, 300), (512, 0), (2048, 1000), (2048, 2047)):
        others = sorted(rng.choice(np.arange(1, POOL), size=T - 1, replace=False).tolist())
        rng.shuffle(others)
        out.append((T, slot, others[:slot] + [0] + others[slot:]))
    return out


def test_moe_layer_logprobs_bitwise_across_compositions(model, pool):
    ref = None
    for T, slot, ids in _compositions():
        log_case(f"235B layer composition T={T} slot={slot}")
        y, lp, tok, tlp = _step(model, pool, ids)
        got = (y[slot].clone(), lp[slot].clone(), tok[slot].clone(), tlp[slot].clone())
        assert bool(torch.isfinite(lp[slot]).all())
        if ref is None:
            ref = got
            continue
        for a, b, what in zip(got, ref, ("layer output", "logprobs", "greedy token", "greedy logprob")):
            assert_bitwise(a, b, f"tracked request {what} at T={T} slot={slot}")
        del y, lp


def test_moe_layer_steps_against_oracle(model, pool):
    """Every library call on the tracked request's row, against the oracle's
    step on the call's own GPU inputs: bf16 outputs within 1e-2 of the row
    scale, fp32 logits / logprobs within 1e-3, the adds bit-exact, the routing
    equal to the order of the library's own logits (and to the oracle's where
    its logits are clearly apart), the greedy token the argmax of the
    library's logprobs row."""
    layer, head = model
    tr = {}
    log_case("235B layer steps vs oracle (tracked request alone)")
    y, lp, tok, tlp = _step(model, pool, [0], trace=tr)
    torch.cuda.synchronize()
    x = f64(pool["x"][:1])
    L = pool["lens"][0]
    g = lambda t: f64(t)
    h, qkv = g(tr["h"]), g(tr["qkv"])
    assert_bf16_close(tr["h"], O.rmsnorm(x, f64(layer.g1), EPS), "rmsnorm 1")
    assert_bf16_close(tr["qkv"], O.gemm(h, f64(layer.w_qkv)), "qkv projection")
    q = qkv[:, :HQ * D].reshape(1, HQ, D)
    kn = qkv[:, HQ * D:(HQ + HKV) * D].reshape(1, HKV, D)
    vn = qkv[:, (HQ + HKV) * D:].reshape(1, HKV, D)
    K0 = np.concatenate([f64(pool["kv0"][0]), kn])
    V0 = np.concatenate([f64(pool["kv0"][1]), vn])
    assert K0.shape[0] == L + 1
    ro, _ = O.decode_attention(q, [K0], [V0], layer.scale)
    assert_bf16_close(tr["attn"][0], ro[0], "decode attention 64/4")
    a = g(tr["attn"]).reshape(1, HQ * D)
    assert_bf16_close(tr["c"], O.gemm(a, f64(layer.w_o)), "o projection")
    r = g(tr["r"])
    assert np.array_equal(r, O.round_bf16(x + g(tr["c"]))), "residual add 1 not bit-exact"
    assert_bf16_close(tr["h2"], O.rmsnorm(r, f64(layer.g2), EPS), "rmsnorm 2")
    h2 = g(tr["h2"])
    ex, wt, lg = O.moe_route(h2, f64(layer.w_gate), K)
    assert_f32_close(tr["logits"], lg, "router logits")
    ids = tr["ids"][0].cpu().numpy()
    mine = g(tr["logits"])[0]
    assert ids.tolist() == sorted(range(E), key=lambda e: (-mine[e], e))[:K], "routing = order of own logits"
    top = -np.sort(-lg[0])[:K + 1]
    if np.all(-np.diff(top) > 1e-3):
        assert ids.tolist() == ex[0].tolist(), "routing = oracle's where its logits are apart"
    z = mine[ids]
    p = np.exp(z - z.max())
    assert np.max(np.abs(g(tr["wts"])[0] - p / p.sum())) <= 1e-3
    ups = [f64(layer.w_up[e]) for e in ids]
    downs = [f64(layer.w_down_e[e]) for e in ids]
    ye = O.moe_ffn(h2, np.arange(K)[None, :], g(tr["wts"]), ups, downs)
    assert_bf16_close(tr["e"], ye, "routed experts")
    yy = g(y)
    assert np.array_equal(yy, O.round_bf16(r + g(tr["e"]))), "residual add 2 not bit-exact"
    assert_bf16_close(tr["hf"], O.rmsnorm(yy, f64(head.gamma), EPS), "final rmsnorm")
    hf = g(tr["hf"])
    logits = np.concatenate([O.gemm(hf, f64(head.w[i:i + 16384])) for i in range(0, V, 16384)], axis=1)
    assert_f32_close(lp, O.log_softmax(logits), "logprobs")
    row = lp[0].cpu()
    assert int(tok[0]) == int(torch.argmax(row)), "greedy token = argmax of the logprobs row"
    assert_bitwise(tlp[0], row[int(tok[0])].to(DEV), "greedy logprob = logprobs at the token")
