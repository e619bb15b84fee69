#!/usr/bin/env python3
"""Benchmark of the batch-invariant hot path on one MI355X.

Timed step: one Qwen3-8B-shaped decode step over B = 256 requests (hidden 4096,
GQA 32/8 heads, head_dim 128, paged KV with 16-token pages, per-request KV
lengths uniform in [1, 4096]):
    RMSNorm -> fused QKV GEMM 4096->6144 -> KV append -> decode attention
    -> RMSNorm -> MLP GEMMs 4096->12288->4096
every call going through the C-ABI library.  Inputs are synthetic (seeded
N(0,1) activations/KV, N(0,0.02) weights: no checkpoints are available) and
resident in HBM before timing starts.

Printed: one JSON line.  `value` = algorithmic bytes moved by the step /
step time (GB/s; every kernel of the step is HBM-bound at B <= 256).
`roofline` is for the dominant kernel (decode attention, timed with HIP
events on the launch stream; at B=256 it is a single kernel, below the
1024 (sequence, kv head) threshold a chunk kernel plus a merge kernel).
`kernels` holds per-kernel times at every workload shape (B = 1..256,
the M ~ 2300 GEMMs and chunked prefill of the mixed batch, the 235B-shaped
lm_head + log_softmax (two calls and fused), greedy token + logprob from the
lm_head, and decode attention) as GB/s or
TFLOP/s and fraction of roofline, plus a whole Qwen3-8B-shaped decoder layer
(O projection, residual adds and gated MLP included) at B = 1, 64, 256.  `cpu_baseline` times the fp64 oracle on the host on a sample of
the same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "batch-invariant GEMM/attn/RMSNorm TFLOP/s & GB/s, % roofline, B=1..256"
EPS = 1e-6


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--kernels", choices=["all", "step", "none"], default="all",
                    help="per-kernel table: every workload shape, only the step's B sweep, or none")
    ap.add_argument("--cpu-sample", type=int, default=256, help="requests of the step the oracle computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes 20 times (counter calibration) and exit")
    ap.add_argument("--only", choices=sorted(ONLY), default=None,
                    help="only run one workload --reps times (for rocprofv3 counter runs) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic work

def bytes_rmsnorm(r, h):
    return 4 * r * h + 2 * h


def bytes_gemm(m, n, k, out_bytes=2):
    return 2 * (m * k + n * k) + out_bytes * m * n


def flops_gemm(m, n, k):
    return 2 * m * n * k


def bytes_append(t, hkv, d):
    return 8 * t * hkv * d


def bytes_decode(lens, hq, hkv, d):
    return 4 * hkv * d * sum(lens) + 4 * len(lens) * hq * d


def flops_decode(lens, hq, d):
    return 4 * hq * d * sum(lens)


def flops_prefill(prefixes, chunks, hq, d):
    keys = sum(sum(p + i + 1 for i in range(n)) for p, n in zip(prefixes, chunks))
    return 4 * hq * d * keys


def bytes_moe(expert_ids, num_experts, h, f):
    """Weights of every expert the batch routes to, plus x and y (bf16) and the routing."""
    import numpy as np
    ids = np.asarray(expert_ids).reshape(-1)
    touched = len(set(int(e) for e in ids if 0 <= e < num_experts))
    t = np.asarray(expert_ids).shape[0]
    return touched * 2 * (2 * h * f) + 2 * t * h * 2 + ids.size * 8


def flops_moe(t, k, h, f):
    return 4 * t * k * h * f


def bytes_prefill(prefixes, chunks, hq, hkv, d):
    return sum(4 * hkv * d * (p + n) + 4 * n * hq * d for p, n in zip(prefixes, chunks))


# ---------------------------------------------------------------- timing helpers

def time_fn(torch, fn, reps, warmup=3, per_graph=10):
    """Median / p10 / p90 microseconds per call of fn(i).

    The calls are captured into HIP graphs of `per_graph` back-to-back launches
    (the library only enqueues kernels on the current stream, so it captures),
    and each graph replay is timed with HIP events on that stream, so launch
    gaps of the host do not inflate short kernels."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for r in range(max(1, reps // per_graph) if reps >= per_graph else 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for i in range(per_graph):
                    fn(r * per_graph + i)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for g in graphs:    # every graph replays once untimed
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        for g in graphs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / per_graph)
    ts.sort()
    return ts[len(ts) // 2], ts[len(ts) // 10], ts[(len(ts) * 9) // 10]


def entry(name, us, nbytes=None, flops=None, bound="hbm", extra=None):
    e = {"kernel": name, "us": round(us[0], 2), "us_p10": round(us[1], 2), "us_p90": round(us[2], 2)}
    if nbytes is not None:
        e["GBps"] = round(nbytes / (us[0] * 1e-6) / 1e9, 1)
    if flops is not None:
        e["TFLOPs"] = round(flops / (us[0] * 1e-6) / 1e12, 2)
    t_roof = max((nbytes or 0) / (HBM_PEAK_GBS * 1e9), (flops or 0) / (BF16_PEAK_TFLOPS * 1e12))
    e["bound"] = "mfma" if (flops or 0) / (BF16_PEAK_TFLOPS * 1e12) > (nbytes or 0) / (HBM_PEAK_GBS * 1e9) else "hbm"
    e["frac_roofline"] = round(t_roof / (us[0] * 1e-6), 4)
    if extra:
        e.update(extra)
    return e


# ---------------------------------------------------------------- the decode step

class DecodeStep:
    """Qwen3-8B-shaped decode step over the first B requests of the workload."""

    HQ, HKV, D, H, QKV, MLP = 32, 8, 128, 4096, 6144, 12288

    def __init__(self, torch, bi, W, B, dev="cuda"):
        self.torch, self.bi, self.B = torch, bi, B
        base = W.SEED_DECODE
        ids = list(range(B))
        self.lens = W.decode_lengths(ids, base)              # cache length incl. the step's new token
        pb = W.allocate_pages(self.lens, base)
        self.kc, self.vc = bi.alloc_kv_cache(pb.num_pages, self.HKV, self.D, 16, dev, fill=0.0)
        # Cache contents: every request's K/V, appended through the library.
        for r0 in range(0, B, 32):
            part = ids[r0:r0 + 32]
            kv = [W.request_kv(r, self.lens[r], self.HKV, self.D, base, device=dev) for r in part]
            lo = sum(self.lens[:r0])
            hi = lo + sum(self.lens[r] for r in part)
            bi.bi_kv_append(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]),
                            pb.slot_mapping[lo:hi].to(dev), self.kc, self.vc)
        self.kv_host = None
        self.bt = pb.block_table.to(dev)
        self.lens_t = torch.tensor(self.lens, dtype=torch.int32, device=dev)
        starts = [0]
        for L in self.lens[:-1]:
            starts.append(starts[-1] + L)
        # slot of each request's newest token (position L - 1)
        self.new_slots = pb.slot_mapping[torch.tensor([s + L - 1 for s, L in zip(starts, self.lens)])].to(dev)
        self.max_len = 4096
        self.x = W.rows_for_requests(ids, self.H, base, device=dev)
        self.g1 = W.randn_bf16((self.H,), base, "gamma", W.WEIGHTS, std=0.1, mean=1.0, device=dev)
        self.g2 = W.randn_bf16((self.H,), base, "gamma", W.WEIGHTS + 1, std=0.1, mean=1.0, device=dev)
        self.w_qkv = W.randn_bf16((self.QKV, self.H), base, "w", W.WEIGHTS + 1, std=0.02, device=dev)
        self.w_up = W.randn_bf16((self.MLP, self.H), base, "w", W.WEIGHTS + 2, std=0.02, device=dev)
        self.w_down = W.randn_bf16((self.H, self.MLP), base, "w", W.WEIGHTS + 3, std=0.02, device=dev)
        e = dict(dtype=torch.bfloat16, device=dev)
        self.h = torch.empty((B, self.H), **e)
        self.qkv = torch.empty((B, self.QKV), **e)
        self.attn = torch.empty((B, self.HQ, self.D), **e)
        self.h2 = torch.empty((B, self.H), **e)
        self.up = torch.empty((B, self.MLP), **e)
        self.down = torch.empty((B, self.H), **e)
        self.lse = torch.empty((B, self.HQ), dtype=torch.float32, device=dev)
        nws = bi.bi_attn_decode_workspace_bytes(B, self.HQ, self.D, self.max_len)
        self.ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
        self.q = self.qkv[:, :4096].view(B, self.HQ, self.D)
        self.k = self.qkv[:, 4096:5120].view(B, self.HKV, self.D)
        self.v = self.qkv[:, 5120:].view(B, self.HKV, self.D)
        self.scale = 1.0 / math.sqrt(self.D)

    def rmsnorm1(self):
        self.bi.bi_rmsnorm(self.x, self.g1, EPS, out=self.h)

    def gemm_qkv(self):
        self.bi.bi_gemm(self.h, self.w_qkv, out=self.qkv)

    def append(self):
        self.bi.bi_kv_append(self.k, self.v, self.new_slots, self.kc, self.vc)

    def attend(self):
        self.bi.bi_attn_decode(self.q, self.kc, self.vc, self.bt, self.lens_t, self.max_len, self.scale,
                               out=self.attn, lse=self.lse, workspace=self.ws)

    def rmsnorm2(self):
        self.bi.bi_rmsnorm(self.attn.view(self.B, self.H), self.g2, EPS, out=self.h2)

    def gemm_up(self):
        self.bi.bi_gemm(self.h2, self.w_up, out=self.up)

    def gemm_down(self):
        self.bi.bi_gemm(self.up, self.w_down, out=self.down)

    def step(self, ev=None):
        self.rmsnorm1()
        self.gemm_qkv()
        self.append()
        if ev is not None:
            ev[0].record()
        self.attend()
        if ev is not None:
            ev[1].record()
        self.rmsnorm2()
        self.gemm_up()
        self.gemm_down()

    def step_bytes(self):
        B = self.B
        return (2 * bytes_rmsnorm(B, self.H) + bytes_gemm(B, self.QKV, self.H) + bytes_append(B, self.HKV, self.D)
                + bytes_decode(self.lens, self.HQ, self.HKV, self.D) + bytes_gemm(B, self.MLP, self.H)
                + bytes_gemm(B, self.H, self.MLP))

    def step_flops(self):
        B = self.B
        return (flops_gemm(B, self.QKV, self.H) + flops_gemm(B, self.MLP, self.H) + flops_gemm(B, self.H, self.MLP)
                + flops_decode(self.lens, self.HQ, self.D))


# ---------------------------------------------------------------- the mixed-batch step

class MixedStep:
    """Qwen3-8B-shaped chunked-prefill + decode step: 4 prefill chunks of 512
    tokens over the seeded prefixes and 252 decode requests with seeded KV
    lengths in [1, 8192], in one batch of M = 2300 rows.  RMSNorm, QKV GEMM, KV
    append (all 2300 new tokens), chunked prefill (the 2048 chunk rows), decode
    (the 252 decode rows), RMSNorm, MLP GEMMs; q/k/v are strided views of the
    QKV output.  Weights are the decode step's."""

    D_DEC = 252

    def __init__(self, torch, bi, W, step, dev="cuda"):
        self.torch, self.bi, self.step = torch, bi, step
        base = W.SEED_MIXED
        self.prefixes = [W.rand_int(0, 8192, base, "len", 100 + s) for s in range(4)]
        self.dlens = W.decode_lengths(range(1000, 1000 + self.D_DEC), base, 1, 8192)
        lens = [p + 512 for p in self.prefixes] + self.dlens
        pb = W.allocate_pages(lens, base)
        self.kc, self.vc = bi.alloc_kv_cache(pb.num_pages, 8, 128, 16, dev, fill=0.0)
        ids = list(range(4)) + list(range(1000, 1000 + self.D_DEC))
        lo = 0
        for j0 in range(0, len(ids), 32):
            part = list(range(j0, min(len(ids), j0 + 32)))
            kv = [W.request_kv(ids[j], lens[j], 8, 128, base, device=dev) for j in part]
            hi = lo + sum(lens[j] for j in part)
            bi.bi_kv_append(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]),
                            pb.slot_mapping[lo:hi].to(dev), self.kc, self.vc)
            lo = hi
            del kv
        starts = [0]
        for L in lens[:-1]:
            starts.append(starts[-1] + L)
        # slots the step's new tokens go to: each chunk's 512 positions, each decode request's last one
        new = [starts[s] + self.prefixes[s] + i for s in range(4) for i in range(512)]
        new += [starts[4 + r] + self.dlens[r] - 1 for r in range(self.D_DEC)]
        self.new_slots = pb.slot_mapping[torch.tensor(new)].to(dev)
        bt = pb.block_table.to(dev)
        self.bt_pre, self.bt_dec = bt[:4].contiguous(), bt[4:].contiguous()
        self.q_start = torch.tensor([0, 512, 1024, 1536, 2048], dtype=torch.int32, device=dev)
        self.ctx = torch.tensor(self.prefixes, dtype=torch.int32, device=dev)
        self.lens_dec = torch.tensor(self.dlens, dtype=torch.int32, device=dev)
        M = self.M = 2048 + self.D_DEC
        e = dict(dtype=torch.bfloat16, device=dev)
        self.x = W.rows_for_requests(range(M), 4096, base, device=dev)
        self.h, self.qkv = torch.empty((M, 4096), **e), torch.empty((M, 6144), **e)
        self.attn, self.h2 = torch.empty((M, 32, 128), **e), torch.empty((M, 4096), **e)
        self.up, self.down = torch.empty((M, 12288), **e), torch.empty((M, 4096), **e)
        self.ws = torch.empty((bi.bi_attn_decode_workspace_bytes(self.D_DEC, 32, 128, 8192),), dtype=torch.uint8,
                              device=dev)
        self.scale = 1.0 / math.sqrt(128)

    def run(self):
        bi, st = self.bi, self.step
        bi.bi_rmsnorm(self.x, st.g1, EPS, out=self.h)
        bi.bi_gemm(self.h, st.w_qkv, out=self.qkv)
        q = self.qkv[:, :4096].view(self.M, 32, 128)
        bi.bi_kv_append(self.qkv[:, 4096:5120].view(self.M, 8, 128), self.qkv[:, 5120:].view(self.M, 8, 128),
                        self.new_slots, self.kc, self.vc)
        bi.bi_attn_prefill(q[:2048], self.q_start, self.ctx, 512, self.kc, self.vc, self.bt_pre, self.scale,
                           out=self.attn[:2048])
        bi.bi_attn_decode(q[2048:], self.kc, self.vc, self.bt_dec, self.lens_dec, 8192, self.scale,
                          out=self.attn[2048:], workspace=self.ws)
        bi.bi_rmsnorm(self.attn.view(self.M, 4096), st.g2, EPS, out=self.h2)
        bi.bi_gemm(self.h2, st.w_up, out=self.up)
        bi.bi_gemm(self.up, st.w_down, out=self.down)

    def work(self):
        M = self.M
        nbytes = (2 * bytes_rmsnorm(M, 4096) + bytes_gemm(M, 6144, 4096) + bytes_append(M, 8, 128)
                  + bytes_prefill(self.prefixes, [512] * 4, 32, 8, 128) + bytes_decode(self.dlens, 32, 8, 128)
                  + bytes_gemm(M, 12288, 4096) + bytes_gemm(M, 4096, 12288))
        flops = (flops_gemm(M, 6144, 4096) + flops_gemm(M, 12288, 4096) + flops_gemm(M, 4096, 12288)
                 + flops_prefill(self.prefixes, [512] * 4, 32, 128) + flops_decode(self.dlens, 32, 128))
        return nbytes, flops


def mixed_step_line(torch, bi, W, step, steps=10):
    ms = MixedStep(torch, bi, W, step)
    for _ in range(3):
        ms.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ms.run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    nbytes, flops = ms.work()
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    line = {"workload": "Qwen3-8B-shaped mixed step: 4 prefill chunks of 512 tokens over prefixes "
                        f"{ms.prefixes} + {ms.D_DEC} decode requests (KV 1-8192), M = {ms.M} rows",
            "us": round(us, 1), "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "flops": flops, "bytes": nbytes,
            "frac_roofline": round(t_roof / (us * 1e-6), 4)}
    del ms
    torch.cuda.empty_cache()
    return line


# ---------------------------------------------------------------- per-kernel table

def copies(w, total=768 << 20):
    """Rotating weight copies so the 256 MB Infinity Cache cannot serve repeated GEMM launches."""
    n = max(1, min(16, total // (w.numel() * 2)))
    return [w] + [w.clone() for _ in range(n - 1)]


def kernel_table(torch, bi, W, step, reps, everything):
    out = []
    dev = "cuda"
    wq, wu, wd = copies(step.w_qkv), copies(step.w_up), copies(step.w_down)
    for B in (1, 8, 64, 256):
        if B > step.B:
            continue
        lens = step.lens[:B]
        x, h, qkv = step.x[:B], step.h[:B], step.qkv[:B]
        up, h2, down = step.up[:B], step.h2[:B], step.down[:B]
        tag = {"B": B}
        us = time_fn(torch, lambda i=0: bi.bi_rmsnorm(x, step.g1, EPS, out=h), reps)
        out.append(entry("rmsnorm [B,4096]", us, bytes_rmsnorm(B, 4096), extra=tag))
        us = time_fn(torch, lambda i=0: bi.bi_gemm(h, wq[i % len(wq)], out=qkv), reps)
        out.append(entry("gemm qkv 4096->6144", us, bytes_gemm(B, 6144, 4096), flops_gemm(B, 6144, 4096), extra=tag))
        us = time_fn(torch, lambda i=0: bi.bi_gemm(h2, wu[i % len(wu)], out=up), reps)
        out.append(entry("gemm up 4096->12288", us, bytes_gemm(B, 12288, 4096), flops_gemm(B, 12288, 4096), extra=tag))
        us = time_fn(torch, lambda i=0: bi.bi_gemm(up, wd[i % len(wd)], out=down), reps)
        out.append(entry("gemm down 12288->4096", us, bytes_gemm(B, 4096, 12288), flops_gemm(B, 4096, 12288),
                         extra=tag))
        # Each repetition decodes another group of B requests (step.B // B
        # disjoint groups, 2.1 GB of KV together), so the Infinity Cache cannot
        # serve repeats; bytes and flops are the groups' mean.
        ng = max(1, step.B // B)
        grp = [slice(j * B, (j + 1) * B) for j in range(ng)]
        attn, lse = step.attn[:B], step.lse[:B]
        us = time_fn(torch, lambda i=0: bi.bi_attn_decode(step.q[grp[i % ng]], step.kc, step.vc, step.bt[grp[i % ng]],
                                                           step.lens_t[grp[i % ng]], 4096, step.scale, out=attn,
                                                           lse=lse, workspace=step.ws), reps)
        glens = [step.lens[sl] for sl in grp]
        out.append(entry("attn decode 32/8 D128", us, sum(bytes_decode(g, 32, 8, 128) for g in glens) / ng,
                         sum(flops_decode(g, 32, 128) for g in glens) / ng,
                         extra=dict(tag, sum_L=sum(map(sum, glens)) / ng, groups=ng)))
    del wq, wu, wd
    if not everything:
        return out
    torch.cuda.empty_cache()
    # Mixed prefill + decode batch: GEMMs at M = 2048 + decode rows (MFMA-bound), chunked prefill.
    M = 2300
    a = W.rows_for_requests(range(M), 4096, W.SEED_MIXED, device=dev)
    a2 = W.rows_for_requests(range(M), 12288, W.SEED_MIXED, device=dev)
    for name, src, w in (("gemm qkv 4096->6144", a, step.w_qkv), ("gemm up 4096->12288", a, step.w_up),
                         ("gemm down 12288->4096", a2, step.w_down)):
        n, k = w.shape
        c = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        us = time_fn(torch, lambda i=0: bi.bi_gemm(src, w, out=c), max(5, reps // 2))
        out.append(entry(name, us, bytes_gemm(M, n, k), flops_gemm(M, n, k), extra={"M": M}))
    del a, a2
    # RMSNorm over the mixed batch's rows, rotating through copies (> 768 MB in
    # all) so that the Infinity Cache cannot serve repeats, and beside it a plain
    # device copy moving the same bytes the same way: the floor for a pass of
    # this size.
    x0 = W.rows_for_requests(range(M), 4096, W.SEED_MIXED, device=dev)
    ncp = (768 << 20) // x0.nbytes + 1
    xr = [x0] + [x0.clone() for _ in range(ncp - 1)]
    yr = [torch.empty_like(x0) for _ in range(ncp)]
    us = time_fn(torch, lambda i=0: bi.bi_rmsnorm(xr[i % ncp], step.g1, EPS, out=yr[i % ncp]), reps)
    out.append(entry("rmsnorm [2300,4096]", us, bytes_rmsnorm(M, 4096), extra={"rows": M}))
    us = time_fn(torch, lambda i=0: yr[i % ncp].copy_(xr[(i + 1) % ncp]), reps)
    out.append(entry("device copy, the bytes of rmsnorm [2300,4096] (floor)", us, 4 * M * 4096,
                     extra={"rows": M, "kind": "torch copy_, not a library kernel"}))
    del x0, xr, yr
    prefixes = [W.rand_int(0, 8192, W.SEED_MIXED, "len", 100 + s) for s in range(4)]
    chunks = [512] * 4
    total = [p + n for p, n in zip(prefixes, chunks)]
    pb = W.allocate_pages(total, W.SEED_MIXED)
    kc, vc = bi.alloc_kv_cache(pb.num_pages, 8, 128, 16, dev, fill=0.0)
    kv = [W.request_kv(s, L, 8, 128, W.SEED_MIXED, device=dev) for s, L in enumerate(total)]
    bi.bi_kv_append(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]), pb.slot_mapping.to(dev), kc, vc)
    del kv
    qp = W.randn_bf16((2048, 32, 128), W.SEED_MIXED, "q", 0, device=dev)
    op = torch.empty_like(qp)
    qs = torch.tensor([0, 512, 1024, 1536, 2048], dtype=torch.int32, device=dev)
    ctx = torch.tensor(prefixes, dtype=torch.int32, device=dev)
    btp = pb.block_table.to(dev)
    us = time_fn(torch, lambda i=0: bi.bi_attn_prefill(qp, qs, ctx, 512, kc, vc, btp, 1 / math.sqrt(128), out=op),
                 max(5, reps // 2))
    out.append(entry("attn prefill 4x512 32/8 D128", us, bytes_prefill(prefixes, chunks, 32, 8, 128),
                     flops_prefill(prefixes, chunks, 32, 128), extra={"prefixes": prefixes}))
    del kc, vc, qp, op
    torch.cuda.empty_cache()
    # Qwen3-235B-shaped: lm_head 4096->151936 (fp32 logits) + log_softmax, separately and fused;
    # decode attention 64/4.
    V = 151936
    wl = W.randn_bf16((V, 4096), W.SEED_MOE, "w", W.WEIGHTS, std=0.02, device=dev)
    for T in (1, 64, 512, 2048):
        ht = W.rows_for_requests(range(T), 4096, W.SEED_MOE, device=dev)
        z = torch.empty((T, V), dtype=torch.float32, device=dev)
        us = time_fn(torch, lambda i=0: bi.bi_gemm(ht, wl, out=z), max(5, reps // 4))
        out.append(entry("gemm lm_head 4096->151936 fp32", us, bytes_gemm(T, V, 4096, 4), flops_gemm(T, V, 4096),
                         extra={"T": T}))
        lp = torch.empty_like(z)
        us = time_fn(torch, lambda i=0: bi.bi_log_softmax(z, out=lp), max(5, reps // 4))
        out.append(entry("log_softmax [T,151936] fp32", us, 8 * T * V, extra={"T": T}))
        # The same two steps fused (bi_lm_head_logprobs): algorithmic work is the
        # GEMM's with the logprobs as its fp32 output.
        lws = torch.empty((bi.lm_head_logprobs_workspace_bytes(T, V),), dtype=torch.uint8, device=dev)
        us = time_fn(torch, lambda i=0: bi.bi_lm_head_logprobs(ht, wl, out=lp, workspace=lws), max(5, reps // 4))
        out.append(entry("lm_head+log_softmax fused 4096->151936 fp32", us, bytes_gemm(T, V, 4096, 4),
                         flops_gemm(T, V, 4096), extra={"T": T}))
        # Greedy sampling (bi_lm_head_greedy): the token and its logprob, no logits
        # written; algorithmic work is the operands read plus 8 bytes per row.
        gws = torch.empty((bi.lm_head_greedy_workspace_bytes(T, V),), dtype=torch.uint8, device=dev)
        tok = torch.empty((T,), dtype=torch.int32, device=dev)
        tlp = torch.empty((T,), dtype=torch.float32, device=dev)
        us = time_fn(torch, lambda i=0: bi.bi_lm_head_greedy(ht, wl, token=tok, logprob=tlp, workspace=gws),
                     max(5, reps // 4))
        out.append(entry("lm_head greedy token+logprob 4096->151936", us, 2 * (T * 4096 + V * 4096) + 8 * T,
                         flops_gemm(T, V, 4096), extra={"T": T}))
        del ht, z, lp, lws, gws, tok, tlp
    del wl
    torch.cuda.empty_cache()
    # Routed experts: 128 experts, top-8, 4096->1536->4096.  Each timed launch
    # uses another routing set, so repeats cannot be served from the Infinity Cache.
    E, K8, F = 128, 8, 1536
    w_up, w_down = W.moe_weights(E, 4096, F, W.SEED_MOE, device=dev)
    w_gate = W.randn_bf16((E, 4096), W.SEED_MOE, "gate", W.WEIGHTS, std=0.02, device=dev)
    for T in (1, 64, 512, 2048):
        sets = 16 if T == 1 else 2
        xs, rts = [], []
        for r in range(sets):
            ids = range(r * T, (r + 1) * T)
            xs.append(W.rows_for_requests(ids, 4096, W.SEED_MOE, device=dev))
            ex, wt = W.moe_routing(ids, E, K8, W.SEED_MOE)
            rts.append((ex.to(dev), wt.to(dev), ex))
        y = torch.empty((T, 4096), dtype=torch.bfloat16, device=dev)
        mws = torch.empty((bi.moe_workspace_bytes(T, K8, E, 4096, F),), dtype=torch.uint8, device=dev)
        us = time_fn(torch, lambda i=0: bi.bi_moe_ffn(xs[i % sets], rts[i % sets][0], rts[i % sets][1], w_up, w_down,
                                                      out=y, workspace=mws), max(5, reps // 4))
        nbytes = sum(bytes_moe(r[2].numpy(), E, 4096, F) for r in rts) / sets
        out.append(entry("moe experts 128x(4096->1536->4096) top-8", us, nbytes, flops_moe(T, K8, 4096, F),
                         extra={"T": T}))
        # The router (gate GEMM 4096->128 with fp32 logits, top-8, softmax weights),
        # and router + experts as one routed layer.
        ids_r = torch.empty((T, K8), dtype=torch.int32, device=dev)
        wts_r = torch.empty((T, K8), dtype=torch.float32, device=dev)
        lg_r = torch.empty((T, E), dtype=torch.float32, device=dev)
        us = time_fn(torch, lambda i=0: bi.bi_moe_route(xs[i % sets], w_gate, K8, logits=lg_r, expert_ids=ids_r,
                                                         expert_weights=wts_r), max(5, reps // 4))
        out.append(entry("moe router 4096->128 top-8", us, 2 * (T * 4096 + E * 4096) + 4 * T * E + 8 * T * K8,
                         flops_gemm(T, E, 4096), extra={"T": T}))

        def routed(i=0):
            bi.bi_moe_route(xs[i % sets], w_gate, K8, logits=lg_r, expert_ids=ids_r, expert_weights=wts_r)
            bi.bi_moe_ffn(xs[i % sets], ids_r, wts_r, w_up, w_down, out=y, workspace=mws)

        routed()
        torch.cuda.synchronize()
        used = ids_r.cpu().numpy()
        us = time_fn(torch, routed, max(5, reps // 4))
        out.append(entry("moe layer routed (router + experts)", us,
                         bytes_moe(used, E, 4096, F) + 2 * E * 4096 + 4 * T * E, flops_moe(T, K8, 4096, F)
                         + flops_gemm(T, E, 4096), extra={"T": T}))
        del xs, rts, y, mws, ids_r, wts_r, lg_r
    del w_up, w_down, w_gate
    torch.cuda.empty_cache()
    # 235B-shaped decode (64/4 heads): 256 requests' caches; a repetition at
    # batch B decodes another of 256 // B disjoint groups (bytes: the mean).
    lens = W.decode_lengths(range(256), W.SEED_MOE)
    pb = W.allocate_pages(lens, W.SEED_MOE)
    kc, vc = bi.alloc_kv_cache(pb.num_pages, 4, 128, 16, dev, fill=0.0)
    for r0 in range(0, 256, 64):
        kv = [W.request_kv(r, lens[r], 4, 128, W.SEED_MOE, device=dev) for r in range(r0, r0 + 64)]
        lo = sum(lens[:r0])
        bi.bi_kv_append(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]),
                        pb.slot_mapping[lo:lo + sum(lens[r0:r0 + 64])].to(dev), kc, vc)
        del kv
    q = W.randn_bf16((256, 64, 128), W.SEED_MOE, "q", 0, device=dev)
    o = torch.empty_like(q)
    btd, lt = pb.block_table.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = torch.empty((bi.bi_attn_decode_workspace_bytes(256, 64, 128, 4096),), dtype=torch.uint8, device=dev)
    for B in (1, 64, 256):
        ng = 256 // B
        grp = [slice(j * B, (j + 1) * B) for j in range(ng)]
        us = time_fn(torch, lambda i=0: bi.bi_attn_decode(q[grp[i % ng]], kc, vc, btd[grp[i % ng]], lt[grp[i % ng]],
                                                           4096, 1 / math.sqrt(128), out=o[:B], workspace=ws), reps)
        glens = [lens[sl] for sl in grp]
        out.append(entry("attn decode 64/4 D128", us, sum(bytes_decode(g, 64, 4, 128) for g in glens) / ng,
                         sum(flops_decode(g, 64, 128) for g in glens) / ng,
                         extra={"B": B, "sum_L": sum(map(sum, glens)) / ng, "groups": ng}))
    del kc, vc, q, o, ws
    torch.cuda.empty_cache()
    # Long-context decode (32/8 heads, D 128): the tracked request at KV 32768
    # co-batched with B - 1 requests of seeded lengths in [1, 32768].
    n_long = 256
    lens = [32768] + W.decode_lengths(range(1, n_long), W.SEED_LONG, 1, 32768)
    pb = W.allocate_pages(lens, W.SEED_LONG)
    kc, vc = bi.alloc_kv_cache(pb.num_pages, 8, 128, 16, dev, fill=0.0)
    lo = 0
    for r0 in range(0, n_long, 16):
        part = range(r0, min(n_long, r0 + 16))
        kv = [W.request_kv(r, lens[r], 8, 128, W.SEED_LONG, device=dev) for r in part]
        hi = lo + sum(lens[r] for r in part)
        bi.bi_kv_append(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]), pb.slot_mapping[lo:hi].to(dev),
                        kc, vc)
        lo = hi
        del kv
    q = W.randn_bf16((n_long, 32, 128), W.SEED_LONG, "q", 0, device=dev)
    o = torch.empty_like(q)
    btd, lt = pb.block_table.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = torch.empty((bi.bi_attn_decode_workspace_bytes(n_long, 32, 128, 32768),), dtype=torch.uint8, device=dev)
    # B = 1 rotates over the four longest requests (the tracked one and three
    # others of 31 K+), the larger batches over disjoint groups, so repeats are
    # not served from the Infinity Cache (bytes: the mean of the groups used).
    longest = sorted(range(n_long), key=lambda r: -lens[r])[:4]
    for B in (1, 16, 64, 256):
        grp = [[r] for r in longest] if B == 1 else [list(range(j * B, (j + 1) * B)) for j in range(n_long // B)]
        idx = [torch.tensor(g_, device=dev) for g_ in grp]
        ng = len(grp)
        qs_ = [q[ix] for ix in idx]
        bts_ = [btd[ix].contiguous() for ix in idx]
        lts_ = [lt[ix] for ix in idx]
        us = time_fn(torch, lambda i=0: bi.bi_attn_decode(qs_[i % ng], kc, vc, bts_[i % ng], lts_[i % ng], 32768,
                                                           1 / math.sqrt(128), out=o[:B], workspace=ws),
                     max(5, reps // 4))
        glens = [[lens[r] for r in g_] for g_ in grp]
        out.append(entry("attn decode long-context 32/8 D128", us, sum(bytes_decode(g_, 32, 8, 128) for g_ in glens)
                         / ng, sum(flops_decode(g_, 32, 128) for g_ in glens) / ng,
                         extra={"B": B, "sum_L": sum(map(sum, glens)) / ng, "groups": ng}))
        del qs_, bts_, lts_
    del kc, vc, q, o, ws
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- whole decoder layer

def bytes_layer(B, lens, h=4096, hq=32, hkv=8, d=128, f=12288):
    """Algorithmic bytes of one decode-layer call: each call's own operands, the
    residual adds and the gated activation fused into the GEMMs before them
    (the O and down projections also read x and write y; the gate/up
    projection writes only silu(gate) * up)."""
    qkv = (hq + 2 * hkv) * d
    return (2 * bytes_rmsnorm(B, h) + bytes_gemm(B, qkv, h) + bytes_append(B, hkv, d)
            + bytes_decode(lens, hq, hkv, d) + bytes_gemm(B, h, hq * d) + 2 * B * h
            + 2 * (B * h + 2 * f * h) + 2 * B * f + bytes_gemm(B, h, f) + 2 * B * h)


def layer_table(torch, bi, W, step, reps):
    """A whole Qwen3-8B-shaped decoder layer (invariant_bi_rmsnorm_02_amd.layer:
    QKV, attention, O projection + residual, gated MLP + residual, the
    residual adds and the gated activation in the GEMM epilogues) decoding the
    first B requests of the step's caches, and the two standalone pointwise
    kernels."""
    from invariant_bi_rmsnorm_02_amd.layer import DecoderLayer
    dev, base = "cuda", W.SEED_DECODE
    w_o = W.randn_bf16((4096, 4096), base, "w", W.WEIGHTS + 4, std=0.02, device=dev)
    w_gu = W.randn_bf16((2 * 12288, 4096), base, "w", W.WEIGHTS + 5, std=0.02, device=dev)
    layer = DecoderLayer(step.w_qkv, w_o, w_gu, step.w_down, step.g1, step.g2, 32, 8, 128, EPS)
    out = []
    for B in (1, 64, 256):
        if B > step.B:
            continue
        x, bt, lt, slots = step.x[:B], step.bt[:B], step.lens_t[:B], step.new_slots[:B]
        us = time_fn(torch, lambda i=0: layer.decode(x, step.kc, step.vc, bt, lt, slots, step.max_len,
                                                     workspace=step.ws), max(10, reps // 2))
        e = entry("decoder layer decode (Qwen3-8B, 9 launches)", us, bytes_layer(B, step.lens[:B]),
                  extra={"B": B, "sum_L": sum(step.lens[:B])})
        e["tokens_per_s_per_layer"] = round(B / (us[0] * 1e-6), 1)
        out.append(e)
    B = step.B
    gu = W.rows_for_requests(range(B), 2 * 12288, base, device=dev)
    m = torch.empty((B, 12288), dtype=torch.bfloat16, device=dev)
    us = time_fn(torch, lambda i=0: bi.bi_silu_mul(gu, out=m), reps)
    out.append(entry("silu_mul [B,2x12288]", us, 6 * B * 12288, extra={"B": B}))
    y = torch.empty_like(step.x)
    us = time_fn(torch, lambda i=0: bi.bi_add(step.x, step.h, out=y), reps)
    out.append(entry("add [B,4096]", us, 6 * B * 4096, extra={"B": B}))
    del layer, w_o, w_gu, gu, m, y
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- cost of invariance

def cost_of_invariance(torch, bi, step, reps):
    """Each op of the decode step at B = 1, 8, 64, 256: libbi.so against the
    shape-adaptive comparator of libbi_adaptive.so (split-K GEMM, fixed
    split-count decode, split-reduction RMSNorm) on the same inputs.  cost =
    t_invariant / t_adaptive - 1; mismatched = output elements whose bits
    differ from libbi.so's (which are the same at every batch size)."""
    from invariant_bi_rmsnorm_02_amd import adaptive as A
    dev = "cuda"
    out = []

    def mism(a, b):
        torch.cuda.synchronize()
        return int((a.view(torch.int16) != b.view(torch.int16)).sum().item())

    wq, wu, wd = copies(step.w_qkv), copies(step.w_up), copies(step.w_down)
    for B in (1, 8, 64, 256):
        if B > step.B:
            continue
        x, h = step.x[:B], step.h[:B]
        ha = torch.empty_like(h)
        wsn = torch.empty((max(256, A.lib().bia_rmsnorm_workspace_bytes(B, 4096)),), dtype=torch.uint8, device=dev)
        ti = time_fn(torch, lambda i=0: bi.bi_rmsnorm(x, step.g1, EPS, out=h), reps)
        ta = time_fn(torch, lambda i=0: A.bia_rmsnorm(x, step.g1, EPS, out=ha, workspace=wsn), reps)
        out.append({"op": "rmsnorm [B,4096]", "B": B, "us_invariant": round(ti[0], 2), "us_adaptive": round(ta[0], 2),
                    "cost": round(ti[0] / ta[0] - 1, 3), "splits": A.rmsnorm_slices(B, 4096),
                    "mismatched": mism(ha, h), "elements": ha.numel()})
        for name, src, ws_, dst in (("gemm qkv 4096->6144", h, wq, step.qkv[:B]),
                                    ("gemm up 4096->12288", step.h2[:B], wu, step.up[:B]),
                                    ("gemm down 12288->4096", step.up[:B], wd, step.down[:B])):
            n, k = ws_[0].shape
            da = torch.empty_like(dst)
            wsg = torch.empty((max(256, A.lib().bia_gemm_workspace_bytes(B, n, k)),), dtype=torch.uint8, device=dev)
            ti = time_fn(torch, lambda i=0: bi.bi_gemm(src, ws_[i % len(ws_)], out=dst), reps)
            ta = time_fn(torch, lambda i=0: A.bia_gemm(src, ws_[i % len(ws_)], out=da, workspace=wsg), reps)
            bi.bi_gemm(src, ws_[0], out=dst)
            A.bia_gemm(src, ws_[0], out=da, workspace=wsg)
            out.append({"op": name, "B": B, "us_invariant": round(ti[0], 2), "us_adaptive": round(ta[0], 2),
                        "cost": round(ti[0] / ta[0] - 1, 3), "splits": A.gemm_splits(B, n, k),
                        "mismatched": mism(da, dst), "elements": da.numel()})
        q, attn = step.q[:B], step.attn[:B]
        aa = torch.empty_like(attn)
        bt, lt = step.bt[:B], step.lens_t[:B]
        wsa = torch.empty((A.lib().bia_attn_decode_workspace_bytes(B, 32, 8, 128, 4096, 16),), dtype=torch.uint8,
                          device=dev)
        ti = time_fn(torch, lambda i=0: bi.bi_attn_decode(q, step.kc, step.vc, bt, lt, 4096, step.scale, out=attn,
                                                          workspace=step.ws), reps)
        ta = time_fn(torch, lambda i=0: A.bia_attn_decode(q, step.kc, step.vc, bt, lt, 4096, step.scale, out=aa,
                                                          workspace=wsa), reps)
        out.append({"op": "attn decode 32/8 D128", "B": B, "us_invariant": round(ti[0], 2),
                    "us_adaptive": round(ta[0], 2), "cost": round(ti[0] / ta[0] - 1, 3),
                    "split_keys": A.decode_split_keys(B, 8, 4096, 16), "mismatched": mism(aa, attn),
                    "elements": aa.numel()})
    del wq, wu, wd
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- HBM traffic (rocprofv3 counters)

COUNTERS_MD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "decode_step_b256_hbm_counters.md")
DECODE_SOURCES = ["attn_decode.hip", "attn_decode_impl.hpp", "attn_chunk.hpp", "kv_layout.hpp", "bi_common.hpp"]


def decode_traffic():
    """HBM bytes per bi_attn_decode launch from the committed FETCH_SIZE / WRITE_SIZE
    summary (calibrated against a plain copy), or None when the decode sources have
    changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(COUNTERS_MD).read()
    except OSError:
        return None
    m = re.search(r"traffic bi_attn_decode bytes_per_launch=(\d+) sources_sha256_16=([0-9a-f]+)", text)
    if not m:
        return None
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "invariant_bi_rmsnorm_02_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return int(m.group(1)) if h.hexdigest()[:16] == m.group(2) else None


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(torch, W, step, sample, min_seconds=10.0, max_reps=50):
    """The fp64 oracle, as it stands, on requests 0..sample-1 of the same decode
    step, repeated until about `min_seconds` of host time have been spent."""
    import numpy as np
    from oracle import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    S = min(sample, step.B)

    def f64(t):
        t = t.detach().cpu()
        return O.bf16_to_f64(t.contiguous().view(torch.int16).numpy())

    x = f64(step.x[:S])
    g1, g2 = f64(step.g1), f64(step.g2)
    wq, wu, wd = f64(step.w_qkv), f64(step.w_up), f64(step.w_down)
    kv = [W.request_kv(r, step.lens[r], 8, 128, W.SEED_DECODE, device="cuda") for r in range(S)]
    ks = [f64(k) for k, _ in kv]
    vs = [f64(v) for _, v in kv]
    del kv

    def one_step():
        h = O.rmsnorm(x, g1, EPS)
        qkv = O.gemm(h, wq)
        q = qkv[:, :4096].reshape(S, 32, 128)
        # the step's new token is position L - 1 of each request's cache
        for r in range(S):
            ks[r][-1] = qkv[r, 4096:5120].reshape(8, 128)
            vs[r][-1] = qkv[r, 5120:].reshape(8, 128)
        o, _ = O.decode_attention(q, ks, vs, 1.0 / math.sqrt(128))
        h2 = O.rmsnorm(o.reshape(S, 4096), g2, EPS)
        O.gemm(O.gemm(h2, wu), wd)

    reps, t0 = 0, time.perf_counter()
    while True:
        one_step()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    lens = step.lens[:S]
    nbytes = (2 * bytes_rmsnorm(S, 4096) + bytes_gemm(S, 6144, 4096) + bytes_append(S, 8, 128)
              + bytes_decode(lens, 32, 8, 128) + bytes_gemm(S, 12288, 4096) + bytes_gemm(S, 4096, 12288))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(nbytes * reps / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": model,
            "seconds": round(dt, 2), "reps": reps, "ms_per_step": round(dt / reps * 1e3, 1),
            "sample": f"the decode step for requests 0-{S - 1} of {step.B} (all weights, their KV caches), "
                      f"fp64 numpy oracle, repeated {reps} times; rate = algorithmic bytes / oracle seconds"}


# ---------------------------------------------------------------- single workloads for counter runs

ONLY = {
    "gemm-up-m2300": "up GEMM 4096->12288 at M=2300 (mixed batch), bf16 out",
    "gemm-up-m256": "up GEMM 4096->12288 at M=256 (decode step), bf16 out",
    "prefill-4x512": "chunked prefill, 4 x 512 tokens over the seeded prefixes, 32/8 heads, D=128",
    "prefill-1x4096": "chunked prefill, 1 x 512 tokens over a 4096-token prefix, 32/8 heads, D=128",
    "prefill-4x4096": "chunked prefill, 4 x 512 tokens over 4096-token prefixes, 32/8 heads, D=128",
    "rmsnorm-2300": "RMSNorm [2300, 4096]",
    "lm-head-t2048": "fused lm_head + log_softmax, T=2048, vocab 151936",
    "layer-decode-b1": "Qwen3-8B-shaped decoder layer, decode of 1 request",
    "layer-decode-b256": "Qwen3-8B-shaped decoder layer, decode of 256 requests (the decode-step caches)",
    "moe-t2048": "routed experts, 128 x (4096->1536->4096) top-8, T=2048",
    "mixed-step": "Qwen3-8B-shaped mixed step: 4 x 512 prefill tokens + 252 decode requests, M=2300",
}


def run_only(torch, bi, W, what, reps):
    """Build one workload of the per-kernel table and launch it `reps` times."""
    dev = "cuda"
    print(f"[bench] only {what}: {ONLY[what]}, {reps} launches", file=sys.stderr, flush=True)
    if what.startswith("gemm-up"):
        M = 2300 if what.endswith("m2300") else 256
        w = W.randn_bf16((12288, 4096), W.SEED_DECODE, "w", W.WEIGHTS + 2, std=0.02, device=dev)
        a = W.rows_for_requests(range(M), 4096, W.SEED_MIXED, device=dev)
        c = torch.empty((M, 12288), dtype=torch.bfloat16, device=dev)
        fn = lambda: bi.bi_gemm(a, w, out=c)
    elif what.startswith("prefill-"):
        if what == "prefill-4x512":
            prefixes = [W.rand_int(0, 8192, W.SEED_MIXED, "len", 100 + s) for s in range(4)]
        else:
            prefixes = [4096] * int(what.split("-")[1].split("x")[0])
        ns = len(prefixes)
        total = [p + 512 for p in prefixes]
        pb = W.allocate_pages(total, W.SEED_MIXED)
        kc, vc = bi.alloc_kv_cache(pb.num_pages, 8, 128, 16, dev, fill=0.0)
        kv = [W.request_kv(s, L, 8, 128, W.SEED_MIXED, device=dev) for s, L in enumerate(total)]
        bi.bi_kv_append(torch.cat([k for k, _ in kv]), torch.cat([v for _, v in kv]), pb.slot_mapping.to(dev),
                        kc, vc)
        qp = W.randn_bf16((512 * ns, 32, 128), W.SEED_MIXED, "q", 0, device=dev)
        op = torch.empty_like(qp)
        qs = torch.tensor([512 * i for i in range(ns + 1)], dtype=torch.int32, device=dev)
        ctx = torch.tensor(prefixes, dtype=torch.int32, device=dev)
        btp = pb.block_table.to(dev)
        fn = lambda: bi.bi_attn_prefill(qp, qs, ctx, 512, kc, vc, btp, 1 / math.sqrt(128), out=op)
    elif what.startswith("layer-decode"):
        from invariant_bi_rmsnorm_02_amd.layer import DecoderLayer
        step = DecodeStep(torch, bi, W, int(what.rsplit("b", 1)[1]))
        w_o = W.randn_bf16((4096, 4096), W.SEED_DECODE, "w", W.WEIGHTS + 4, std=0.02, device=dev)
        w_gu = W.randn_bf16((2 * 12288, 4096), W.SEED_DECODE, "w", W.WEIGHTS + 5, std=0.02, device=dev)
        layer = DecoderLayer(step.w_qkv, w_o, w_gu, step.w_down, step.g1, step.g2, 32, 8, 128, EPS)
        fn = lambda: layer.decode(step.x, step.kc, step.vc, step.bt, step.lens_t, step.new_slots, step.max_len,
                                  workspace=step.ws)
    elif what == "moe-t2048":
        E, K8, F, T = 128, 8, 1536, 2048
        w_up, w_down = W.moe_weights(E, 4096, F, W.SEED_MOE, device=dev)
        x = W.rows_for_requests(range(T), 4096, W.SEED_MOE, device=dev)
        ex, wt = W.moe_routing(range(T), E, K8, W.SEED_MOE)
        ex, wt = ex.to(dev), wt.to(dev)
        y = torch.empty((T, 4096), dtype=torch.bfloat16, device=dev)
        mws = torch.empty((bi.moe_workspace_bytes(T, K8, E, 4096, F),), dtype=torch.uint8, device=dev)
        fn = lambda: bi.bi_moe_ffn(x, ex, wt, w_up, w_down, out=y, workspace=mws)
    elif what == "mixed-step":
        ms = MixedStep(torch, bi, W, DecodeStep(torch, bi, W, 256))
        fn = ms.run
    elif what == "rmsnorm-2300":
        x = W.rows_for_requests(range(2300), 4096, W.SEED_MIXED, device=dev)
        g = W.randn_bf16((4096,), W.SEED_MIXED, "gamma", W.WEIGHTS, std=0.1, mean=1.0, device=dev)
        y = torch.empty_like(x)
        fn = lambda: bi.bi_rmsnorm(x, g, EPS, out=y)
    else:
        V, T = 151936, 2048
        wl = W.randn_bf16((V, 4096), W.SEED_MOE, "w", W.WEIGHTS, std=0.02, device=dev)
        ht = W.rows_for_requests(range(T), 4096, W.SEED_MOE, device=dev)
        lp = torch.empty((T, V), dtype=torch.float32, device=dev)
        lws = torch.empty((bi.lm_head_logprobs_workspace_bytes(T, V),), dtype=torch.uint8, device=dev)
        fn = lambda: bi.bi_lm_head_logprobs(ht, wl, out=lp, workspace=lws)
    torch.cuda.synchronize()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"only": what, "launches": reps}), flush=True)


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported (the path shards by "
              "requests and kv heads with no exchange across GPUs).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_bytes:
        x = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(20):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 20}), flush=True)
        return
    import invariant_bi_rmsnorm_02_amd as bi
    import workloads as W
    if not os.path.exists(bi.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    bi.lib()
    torch.cuda.set_device(0)
    if args.only:
        run_only(torch, bi, W, args.only, args.reps)
        return
    print(f"[bench] building the decode-step workload B={args.batch}", file=sys.stderr, flush=True)
    step = DecodeStep(torch, bi, W, args.batch)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step.step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        step.step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    attn_us = sum(a.elapsed_time(b) for a, b in evs) / args.steps * 1e3
    print(f"[bench] step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms), attention {attn_us:.1f} us",
          file=sys.stderr, flush=True)

    nbytes = step.step_bytes()
    attn_bytes = bytes_decode(step.lens, 32, 8, 128)
    value = nbytes / (ms_step * 1e-3) / 1e9
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Qwen3-8B-shaped decode step: RMSNorm, QKV GEMM 4096->6144, KV append, "
                               f"decode attention 32/8 heads D128 paged (16) KV L~U[1,4096], RMSNorm, "
                               f"MLP GEMMs 4096->12288->4096", "batch": args.batch, "sum_kv_len": sum(step.lens),
                   "step_bytes": nbytes, "step_flops": step.step_flops(), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "bi_attn_decode (decode_order_kernel + attn_decode_queue_kernel: whole-sequence wavefronts from a longest-first work queue, no merge launch at B=256)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": decode_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                                     "profiles/decode_step_b256_hbm_counters.md)",
                     "avg_us": round(attn_us, 2), "algorithmic_bytes": attn_bytes},
    }
    if args.kernels != "none":
        print("[bench] per-kernel table", file=sys.stderr, flush=True)
        result["kernels"] = kernel_table(torch, bi, W, step, args.reps, args.kernels == "all")
        if args.kernels == "all":
            print("[bench] mixed prefill + decode step", file=sys.stderr, flush=True)
            result["mixed_step"] = mixed_step_line(torch, bi, W, step)
        print("[bench] decoder layer", file=sys.stderr, flush=True)
        result["kernels"] += layer_table(torch, bi, W, step, args.reps)
        print("[bench] cost of invariance", file=sys.stderr, flush=True)
        result["cost_of_invariance"] = cost_of_invariance(torch, bi, step, args.reps)
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(torch, W, step, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
