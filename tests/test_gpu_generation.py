"""Greedy generation under random co-batching: the "many completions, how many
unique" measurement of "Defeating Nondeterminism in LLM Inference" (Thinking
Machines Lab, the experiment section), run on a synthetic two-layer
Qwen3-8B-shaped model with random weights instead of the pages' trained
Qwen3-235B (no checkpoints are available).

One tracked request (a fixed 16-token prompt) generates 64 tokens greedily,
again and again.  At every decode step it shares the batch with a random number
of other requests (0..255, each with its own cached length) at a random slot,
so the batch size the kernels see changes from step to step and from run to
run.  With the library every run must give the same tokens and bitwise the same
logprobs.  The shape-adaptive comparator (split-K GEMM, split decode attention
and split RMSNorm, each choosing its split from the batch size) is run the same
way as the negative control: its logprobs change with the co-batch, and its
completions are expected to split into several unique ones.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import bi, ensure_lib, log_case
from invariant_bi_rmsnorm_02_amd.layer import DecoderLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 71
H, HQ, HKV, D, F, V = 4096, 32, 8, 128, 12288, 151936
# BI_GENERATION_RUNS sets the number of completions per side (16 by default;
# the pages' own count, 1000, takes about ten minutes).
LAYERS, PROMPT, GEN, OTHERS = 2, 16, 64, 255
RUNS = int(os.environ.get("BI_GENERATION_RUNS", "16"))
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


class AdaptiveLayer(DecoderLayer):
    """The same layer with its three reductions taken from the shape-adaptive
    comparator library."""

    def _norm(self, x, gamma):
        from invariant_bi_rmsnorm_02_amd import adaptive as A
        return A.bia_rmsnorm(x, gamma, self.eps)

    def _gemm(self, a, w):
        from invariant_bi_rmsnorm_02_amd import adaptive as A
        return A.bia_gemm(a, w)

    def _attend(self, q, k_cache, v_cache, block_table, seq_lens, max_seq_len, workspace):
        from invariant_bi_rmsnorm_02_amd import adaptive as A
        return A.bia_attn_decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, self.scale)[0]


class Model:
    """Embedding -> LAYERS decoder layers -> RMSNorm -> greedy lm_head, over a
    paged cache per layer shared by the tracked request (sequence 0) and
    OTHERS co-batched requests (sequences 1..OTHERS) whose caches hold random
    K/V of random lengths."""

    def __init__(self, adaptive: bool):
        w = lambda n, k, i: W.randn_bf16((n, k), SEED, "w", i, std=0.02, device=DEV)
        g = lambda i: W.randn_bf16((H,), SEED, "gamma", i, std=0.1, mean=1.0, device=DEV)
        cls = AdaptiveLayer if adaptive else DecoderLayer
        self.layers = [cls(w((HQ + 2 * HKV) * D, H, 10 * l + 1), w(H, HQ * D, 10 * l + 2), w(2 * F, H, 10 * l + 3),
                           w(H, F, 10 * l + 4), g(10 * l + 5), g(10 * l + 6), HQ, HKV, D, EPS)
                       for l in range(LAYERS)]
        self.emb = W.randn_bf16((V, H), SEED, "w", 1000, device=DEV)
        self.g_final = g(1001)
        self.w_lm = w(V, H, 1002)
        self.other_lens = [W.rand_int(1, 2048, SEED, "len", i) for i in range(OTHERS)]
        total = [PROMPT + GEN] + [L + 1 for L in self.other_lens]
        pb = W.allocate_pages(total, SEED)
        self.bt = pb.block_table.to(DEV)
        starts = np.cumsum([0] + total[:-1]).tolist()
        sm = pb.slot_mapping
        self.track_slots = sm[:PROMPT + GEN].to(DEV)
        self.other_new_slot = torch.stack([sm[st + L] for st, L in zip(starts[1:], self.other_lens)]).to(DEV)
        self.caches = []
        for _ in range(LAYERS):
            kc, vc = bi.alloc_kv_cache(pb.num_pages, HKV, D, 16, fill=0.0)
            self.caches.append((kc, vc))
        for s, L in enumerate(self.other_lens):
            k, v = W.request_kv(s + 1, L, HKV, D, SEED, device=DEV)
            slots = sm[starts[s + 1]:starts[s + 1] + L].to(DEV)
            for kc, vc in self.caches:
                bi.bi_kv_append(k, v, slots, kc, vc)
        nws = bi.bi_attn_decode_workspace_bytes(OTHERS + 1, HQ, D, 2048 + 1)
        self.ws = torch.empty((nws,), dtype=torch.uint8, device=DEV)
        self.gws = torch.empty((bi.lm_head_greedy_workspace_bytes(OTHERS + 1, V),), dtype=torch.uint8, device=DEV)

    def _head(self, x):
        h = self.layers[0]._norm(x, self.g_final)
        lp = torch.empty((x.shape[0],), dtype=torch.float32, device=DEV)
        return bi.bi_lm_head_greedy(h, self.w_lm, logprob=lp, workspace=self.gws)

    def prefill(self, prompt):
        x = self.emb[prompt]
        qs = torch.tensor([0, PROMPT], dtype=torch.int32, device=DEV)
        ctx = torch.zeros(1, dtype=torch.int32, device=DEV)
        for layer, (kc, vc) in zip(self.layers, self.caches):
            x = layer.prefill(x, kc, vc, self.bt[:1], qs, ctx, self.track_slots[:PROMPT], PROMPT)
        tok, lp = self._head(x[PROMPT - 1:])
        return int(tok[0]), float(lp[0])

    def decode(self, token, pos, others, other_tokens, slot):
        """One decode step of the tracked request (its `pos`-th token, `token`)
        with the co-batched requests `others` (inputs `other_tokens`), the
        tracked row at `slot`."""
        rows, toks = list(others), list(other_tokens)
        rows.insert(slot, -1)
        toks.insert(slot, token)
        idx = torch.tensor([r + 1 for r in rows], dtype=torch.long, device=DEV)
        lens = [pos + 1 if r < 0 else self.other_lens[r] + 1 for r in rows]
        toks = torch.tensor(toks, dtype=torch.long, device=DEV)
        x = self.emb[toks]
        slots = torch.stack([self.track_slots[pos] if r < 0 else self.other_new_slot[r] for r in rows])
        lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
        bt = self.bt[idx].contiguous()
        for layer, (kc, vc) in zip(self.layers, self.caches):
            x = layer.decode(x, kc, vc, bt, lens_t, slots, max(lens), workspace=self.ws)
        tok, lp = self._head(x)
        return int(tok[slot]), lp[slot].clone()


def _generate(model, run):
    prompt = torch.tensor([W.rand_int(0, V - 1, SEED, "misc", i) for i in range(PROMPT)], device=DEV)
    tok, _ = model.prefill(prompt)
    g = np.random.default_rng([SEED, run])
    tokens, lps, sizes = [tok], [], []
    for t in range(GEN - 1):
        k = int(g.integers(0, OTHERS + 1))
        others = sorted(g.choice(OTHERS, size=k, replace=False).tolist())
        other_tokens = g.integers(0, V, size=k).tolist()
        slot = int(g.integers(0, k + 1))
        tok, lp = model.decode(tokens[-1], PROMPT + t, others, other_tokens, slot)
        tokens.append(tok)
        lps.append(lp)
        sizes.append(k + 1)
    return tuple(tokens), torch.stack(lps).view(torch.int32).cpu(), sizes


def _unique(model, what):
    outs = []
    for run in range(RUNS):
        outs.append(_generate(model, run))
        if run < 16 or run % 50 == 0:
            print(f"[gen] {what} run {run}: batch sizes {outs[-1][2][:6]}..., tokens {outs[-1][0][:8]}...", flush=True)
    return outs


def test_greedy_generation_under_random_cobatching():
    log_case(f"generation: {LAYERS} layers, prompt {PROMPT}, {GEN} tokens, {RUNS} runs, library")
    outs = _unique(Model(adaptive=False), "library")
    assert len({o[0] for o in outs}) == 1, "the library's completions differ between co-batches"
    for o in outs[1:]:
        assert torch.equal(o[1], outs[0][1]), "the library's logprobs differ bitwise between co-batches"
    torch.cuda.empty_cache()
    log_case("generation: the shape-adaptive comparator")
    ad = _unique(Model(adaptive=True), "adaptive")
    uniq = len({o[0] for o in ad})
    ref = ad[0][0]
    first = [next((i for i, (a, b) in enumerate(zip(o[0], ref)) if a != b), None) for o in ad[1:]]
    first = sorted(i for i in first if i is not None)
    print(f"[gen] adaptive: completions leave run 0's at tokens {first}", flush=True)
    # the first decode step already sees a different batch size in every run
    lp0 = {int(o[1][0]) for o in ad}
    print(f"[gen] unique completions: library 1 of {RUNS}, adaptive {uniq} of {RUNS}; "
          f"adaptive first-step logprob bit patterns {len(lp0)}", flush=True)
    assert len(lp0) > 1, "negative control: the comparator's logprob did not change with the batch"
    assert uniq > 1, "negative control: the comparator's completions did not split"
