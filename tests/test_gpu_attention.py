"""KV append, decode and chunked-prefill attention on the GPU.

Parity with the fp64 oracle (which sees each request's logical K/V, never the
page table), the pages' worked chunk example, closed forms, and the pages'
property checked bitwise on the GPU: a request's outputs do not depend on the
batch size, its slot, its physical pages, the co-batched load, or whether its
tokens are prefilled or decoded.  Unused cache slots are poisoned with NaN so
any read of a slot past a sequence's end would show up.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import (O, assert_bf16_close, assert_bitwise, assert_f32_close, bi, ensure_lib, f64,
                      log_case)

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


class Batch:
    """Requests over a NaN-poisoned paged cache, filled through bi_kv_append."""

    def __init__(self, requests, seq_lens, hq, hkv, d, base, perm_index=0, page_size=16, extra_pages=3,
                 kv_fn=W.request_kv, q_kind="q"):
        self.requests, self.seq_lens = list(requests), list(seq_lens)
        self.hq, self.hkv, self.d, self.base = hq, hkv, d, base
        self.pb = W.allocate_pages(self.seq_lens, base, page_size, extra_pages, perm_index)
        self.kc, self.vc = bi.alloc_kv_cache(self.pb.num_pages, hkv, d, page_size, fill=NAN)
        self.kv = [kv_fn(r, L, hkv, d, base, device=DEV) for r, L in zip(self.requests, self.seq_lens)]
        if sum(self.seq_lens):
            k_all = torch.cat([k for k, _ in self.kv]).contiguous()
            v_all = torch.cat([v for _, v in self.kv]).contiguous()
            bi.bi_kv_append(k_all, v_all, self.pb.slot_mapping.to(DEV), self.kc, self.vc)
        self.q = torch.stack([W.randn_bf16((hq, d), base, q_kind, r, device=DEV) for r in self.requests]) \
            if self.requests else torch.empty((0, hq, d), dtype=torch.bfloat16, device=DEV)
        self.bt = self.pb.block_table.to(DEV)
        self.lens = torch.tensor(self.seq_lens, dtype=torch.int32, device=DEV)
        self.scale = 1.0 / math.sqrt(d)

    def decode(self, max_seq_len=None, q=None, lens=None, workspace=None):
        msl = max(self.seq_lens) if max_seq_len is None else max_seq_len
        qq = self.q if q is None else q
        lse = torch.empty((qq.shape[0], self.hq), dtype=torch.float32, device=DEV)
        out, lse = bi.bi_attn_decode(qq, self.kc, self.vc, self.bt, self.lens if lens is None else lens, msl,
                                     self.scale, lse=lse, workspace=workspace)
        return out, lse

    def oracle(self, idx):
        """fp64 decode of the listed batch slots."""
        q = f64(self.q[idx])
        ks = [f64(self.kv[i][0]) for i in idx]
        vs = [f64(self.kv[i][1]) for i in idx]
        return O.decode_attention(q, ks, vs, self.scale)


# ---------------------------------------------------------------- KV append

def _tile_positions(off, d):
    """Element offset inside a (page, head) block of in-page token `off`, dim d,
    per the tiled layout documented in include/bi.h (restated here)."""
    t, j = off // 16, off % 16
    slot = 8 * ((j // 4) % 2) + 4 * (j // 8) + j % 4
    k = t * 16 * D_ALL[0] + (d // 8) * 128 + slot * 8 + d % 8
    v = t * 16 * D_ALL[0] + (d // 16) * 256 + (j // 8) * 128 + (d % 16) * 8 + j % 8
    return k, v


D_ALL = [0]


def _run_slots(pages, ps):
    """A chunk-like slot mapping: whole 16-token tiles in order (page-aligned
    and not), runs that start or end mid-tile, a run broken by a padding
    token, a run whose tiles are out of order, and scattered single tokens."""
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(pages, generator=g).tolist()
    base = lambda i: perm[i] * ps
    runs = [list(range(base(0), base(0) + 48)),            # three whole tiles of one page (ps >= 64) or three pages
            list(range(base(1) + 5, base(1) + 40)),        # starts mid-tile
            list(range(base(2), base(2) + 16)),
            list(range(base(3) + 16, base(3) + 16 + 20)),
            [base(4) + 3, base(4) + 1, base(4) + 2]]
    broken = list(range(base(5), base(5) + 32))
    broken[20] = -1                                        # padding inside a tile
    swapped = list(range(base(6), base(6) + 16))
    swapped[3], swapped[4] = swapped[4], swapped[3]        # one tile, tokens out of order
    s = [x for r in runs for x in r] + broken + swapped
    singles = torch.randperm(pages * ps, generator=g).tolist()
    used = set(s)
    s += [x for x in singles if x not in used and x // ps not in perm[:7]][:21]
    return torch.tensor(s, dtype=torch.int32)


@pytest.mark.parametrize("ps,d,kind", [(16, 128, "random"), (64, 128, "random"), (16, 128, "runs"),
                                       (64, 128, "runs"), (16, 64, "runs"), (256, 64, "runs")])
def test_kv_append_layout_bit_exact(ps, d, kind):
    hkv, pages = 8, 40
    D_ALL[0] = d
    slots = torch.randperm(pages * ps, generator=torch.Generator().manual_seed(3))[:300].to(torch.int32) \
        if kind == "random" else _run_slots(pages, ps)
    t = slots.shape[0]
    k_new = W.randn_bf16((t, hkv, d), 1, "k", 0, device=DEV)
    v_new = W.randn_bf16((t, hkv, d), 1, "v", 0, device=DEV)
    if kind == "random":
        slots[7] = -1                                # padding token: skipped
    kc, vc = bi.alloc_kv_cache(pages, hkv, d, ps, fill=0.5)
    bi.bi_kv_append(k_new, v_new, slots.to(DEV), kc, vc)
    ek = torch.full((pages, hkv, ps * d), 0.5, dtype=torch.bfloat16)
    ev = torch.full((pages, hkv, ps * d), 0.5, dtype=torch.bfloat16)
    kh, vh = k_new.cpu(), v_new.cpu()
    dims = np.arange(d)
    for i in range(t):
        s = int(slots[i])
        if s < 0:
            continue
        kpos, vpos = _tile_positions(s % ps, dims)
        ek[s // ps, :, torch.from_numpy(kpos)] = kh[i]
        ev[s // ps, :, torch.from_numpy(vpos)] = vh[i]
    assert_bitwise(kc.cpu().view(pages, hkv, -1), ek, "k cache")
    assert_bitwise(vc.cpu().view(pages, hkv, -1), ev, "v cache")


# ---------------------------------------------------------------- decode: pins

@pytest.mark.parametrize("B", [1, 3, 8])
def test_decode_tiny_workload(B):
    # Single-head decode, head_dim 64, KV lengths {1, 255, 256, 1000}; request 0 tracked.
    lens_cycle = [1000, 1, 255, 256]
    lens = [lens_cycle[i % 4] for i in range(B)]
    log_case(f"decode tiny B={B} lens={lens}")
    bt = Batch(range(B), lens, 1, 1, 64, W.SEED_TINY)
    out, lse = bt.decode()
    ro, rl = bt.oracle(list(range(B)))
    for b in range(B):
        assert_bf16_close(out[b], ro[b], f"tiny decode request {b} L={lens[b]}")
    assert_f32_close(lse, rl, "tiny decode lse")
    one = Batch([0], [1000], 1, 1, 64, W.SEED_TINY)
    o1, l1 = one.decode()
    assert_bitwise(out[0], o1[0], "tiny: request 0 vs B=1")
    assert_bitwise(lse[0], l1[0], "tiny: request 0 lse vs B=1")


def test_decode_single_token_exact():
    bt = Batch(range(4), [1, 1, 1, 1], 32, 8, 128, W.SEED_DECODE)
    out, lse = bt.decode()
    for b in range(4):
        v0 = bt.kv[b][1][0]                          # [Hkv, D]
        assert_bitwise(out[b], v0.repeat_interleave(4, dim=0), f"L=1 output equals v0 (request {b})")
    s = torch.einsum("bhd,bhd->bh", f64t(bt.q), f64t(torch.stack([kv[0][0] for kv in bt.kv]).repeat_interleave(4, 1)))
    assert_f32_close(lse, (s * bt.scale).numpy(), "L=1 lse")


def f64t(t):
    return torch.from_numpy(f64(t))


def test_decode_uniform_and_constant_value_closed_forms():
    L, hkv, hq, d = 700, 2, 8, 128
    bt = Batch([0], [L], hq, hkv, d, 11)
    zero_q = torch.zeros_like(bt.q)
    out, lse = bt.decode(q=zero_q)
    v = f64(bt.kv[0][1])                             # [L, Hkv, D]
    want = np.repeat(v.mean(axis=0), hq // hkv, axis=0)
    assert_bf16_close(out[0], want, "q = 0: mean of V")
    assert_f32_close(lse, np.full((1, hq), math.log(L)), "q = 0: lse = ln L")


def test_decode_chunk_partials_follow_pages_example():
    # 1,000 keys = 256 + 256 + 256 + 232: four partials are written, a fifth
    # (allowed by max_seq_len) is not, and each is equivalent to the oracle's partial.
    L, d = 1000, 64
    bt = Batch([0], [L], 1, 1, d, W.SEED_TINY)
    msl = 1280
    need = bi.bi_attn_decode_workspace_bytes(1, 1, d, msl)
    ws = torch.full((need // 4,), -12345.0, dtype=torch.float32, device=DEV)
    bt.decode(max_seq_len=msl, workspace=ws)
    rec = ws[: 5 * (d + 4)].view(5, d + 4).cpu().double().numpy()
    q = f64(bt.q[0, 0])
    k, v = f64(bt.kv[0][0][:, 0]), f64(bt.kv[0][1][:, 0])
    sizes = O.kv_chunks(L)
    assert sizes == [256, 256, 256, 232]
    start = 0
    for c, size in enumerate(sizes):
        m, l, acc = O.chunk_partial(q, k[start:start + size], v[start:start + size], bt.scale)
        start += size
        # The kernel's partial is relative to its reference max r (raised only
        # when a score passes it by more than 8 in log2 units), so what is fixed
        # is the chunk's log-sum-exp r + ln l, the normalised acc / l, and
        # max - 8 ln 2 <= r <= max.
        r, lk = rec[c, d] * math.log(2.0), rec[c, d + 1]
        assert m - 8 * math.log(2.0) - 1e-3 <= r <= m + 1e-3, f"chunk {c} reference max"
        assert abs((r + math.log(lk)) - (m + math.log(l))) < 1e-3, f"chunk {c} lse"
        rel = np.max(np.abs(rec[c, :d] / lk - acc / l)) / max(np.max(np.abs(acc / l)), 1e-30)
        assert rel < 1e-2, f"chunk {c} acc / l"
    assert np.all(rec[4] == -12345.0), "no fifth partial for a 1,000-token cache"


# ---------------------------------------------------------------- decode: parity

@pytest.mark.parametrize("hq,hkv,B,check", [(32, 8, 8, 8), (32, 8, 64, 6), (64, 4, 8, 8), (16, 16, 4, 4),
                                            (32, 16, 5, 5)])
def test_decode_parity_workload_shapes(hq, hkv, B, check):
    base = W.SEED_DECODE if hq == 32 else W.SEED_MOE
    lens = W.decode_lengths(range(B), base)
    log_case(f"decode parity hq={hq} hkv={hkv} B={B}")
    bt = Batch(range(B), lens, hq, hkv, 128, base)
    out, lse = bt.decode()
    idx = sorted(set(np.linspace(0, B - 1, check).astype(int).tolist()))
    ro, rl = bt.oracle(idx)
    for j, b in enumerate(idx):
        assert_bf16_close(out[b], ro[j], f"request {b} L={lens[b]}")
    assert_f32_close(lse[idx], rl, "lse")


def test_decode_long_context_parity():
    L = 32768
    log_case("decode parity L=32768")
    bt = Batch([0], [L], 32, 8, 128, W.SEED_LONG)
    out, lse = bt.decode()
    ro, rl = bt.oracle([0])
    assert_bf16_close(out[0], ro[0], "L=32768")
    assert_f32_close(lse, rl, "L=32768 lse")


# ---------------------------------------------------------------- decode: invariance

def test_decode_batch_invariance():
    hq, hkv, d = 32, 8, 128
    ref = None
    for B in (1, 8, 64, 256):
        for pos, perm in sorted({(0, 0), (B // 2, 1), (B - 1, 2)}):
            ids = list(range(1, B))
            ids.insert(pos, 0)
            lens = W.decode_lengths(ids, W.SEED_DECODE)
            log_case(f"decode invariance B={B} slot={pos} perm={perm}")
            bt = Batch(ids, lens, hq, hkv, d, W.SEED_DECODE, perm_index=perm)
            out, lse = bt.decode(max_seq_len=4096 if B > 1 else None)
            got = (out[pos].clone(), lse[pos].clone())
            if ref is None:
                ref = got
            assert_bitwise(got[0], ref[0], f"request 0 output at B={B} slot={pos}")
            assert_bitwise(got[1], ref[1], f"request 0 lse at B={B} slot={pos}")


def test_decode_run_to_run():
    bt = Batch(range(16), W.decode_lengths(range(16), 7), 32, 8, 128, 7)
    o0, l0 = bt.decode()
    for _ in range(20):
        o, l = bt.decode()
        assert_bitwise(o, o0, "decode repeat")
        assert_bitwise(l, l0, "decode lse repeat")


def test_decode_growing_cache_with_random_co_batch():
    # One request grows token by token; at every step it is decoded alone and
    # with a random co-batch.  Its output must match bit for bit, and the
    # partial of a finished chunk must not change as the cache grows.
    hq, hkv, d, Lmax = 32, 8, 128, 700
    track = Batch([0], [Lmax], hq, hkv, d, W.SEED_LONG, kv_fn=W.request_kv_prefix_stable)
    others_n = 40
    others_lens = W.decode_lengths(range(1, others_n + 1), W.SEED_LONG, 1, 2000)
    others = Batch(range(1, others_n + 1), others_lens, hq, hkv, d, W.SEED_LONG, perm_index=5)
    rng = np.random.default_rng(4)
    # One joint pool holding the co-batch's pages followed by the tracked request's.
    kc = torch.cat([others.kc, track.kc]).contiguous()
    vc = torch.cat([others.vc, track.vc]).contiguous()
    width = max(others.bt.shape[1], track.bt.shape[1])

    def pad(r):
        return torch.cat([r, torch.full((width - r.shape[0],), -1, dtype=torch.int32, device=DEV)])

    trow = pad(torch.where(track.bt[0] >= 0, track.bt[0] + others.pb.num_pages, track.bt[0]))
    orows = [pad(others.bt[i]) for i in range(others_n)]
    probe = W.randn_bf16((1, hq, d), W.SEED_LONG, "q", 99, device=DEV)
    probe_ref = None
    need = bi.bi_attn_decode_workspace_bytes(1, hq, d, Lmax)
    for L in list(range(1, 40)) + list(range(250, 262)) + list(range(505, 520)) + [600, 699, 700]:
        q = W.randn_bf16((1, hq, d), W.SEED_LONG, "q", 10_000 + L, device=DEV)
        lens1 = torch.tensor([L], dtype=torch.int32, device=DEV)
        o1, l1 = bi.bi_attn_decode(q, track.kc, track.vc, track.bt, lens1, Lmax, track.scale,
                                   lse=torch.empty((1, hq), dtype=torch.float32, device=DEV))
        if L >= 256:
            # chunk-0 partial of a fixed probe query stays bitwise stable as L grows
            ws = torch.zeros((need // 4,), dtype=torch.float32, device=DEV)
            bi.bi_attn_decode(probe, track.kc, track.vc, track.bt, lens1, Lmax, track.scale, workspace=ws)
            rec0 = ws[: d + 4].clone()               # (request 0, q head 0, chunk 0)
            if probe_ref is None:
                probe_ref = rec0
            assert_bitwise(rec0, probe_ref, f"chunk-0 partial at L={L}")
        k = int(rng.integers(0, others_n + 1))
        sel = sorted(rng.choice(others_n, size=k, replace=False).tolist())
        pos = int(rng.integers(0, k + 1))
        qs = [others.q[i:i + 1] for i in sel]
        qs.insert(pos, q)
        lens = [others_lens[i] for i in sel]
        lens.insert(pos, L)
        rows = [orows[i] for i in sel]
        rows.insert(pos, trow)
        btab = torch.stack(rows).contiguous()
        qq = torch.cat(qs).contiguous()
        lse = torch.empty((k + 1, hq), dtype=torch.float32, device=DEV)
        o, l = bi.bi_attn_decode(qq, kc, vc, btab, torch.tensor(lens, dtype=torch.int32, device=DEV),
                                 max(lens + [Lmax]), track.scale, lse=lse)
        assert_bitwise(o[pos], o1[0], f"tracked output at L={L} with {k} co-batched")
        assert_bitwise(l[pos], l1[0], f"tracked lse at L={L} with {k} co-batched")


@pytest.fixture(scope="module")
def long_batch():
    """The long-context workload's requests: request 0 with a 32768-token
    cache, 255 others with seeded lengths in [1, 32768]."""
    lens = [32768] + W.decode_lengths(range(1, 256), W.SEED_LONG, 1, 32768)
    return Batch(range(256), lens, 32, 8, 128, W.SEED_LONG, perm_index=3)


def test_decode_long_context_co_batch_invariance(long_batch):
    """The long-context workload at its size: one request at KV 32768 (and at
    20001, a partial last chunk) decoded alone and among 15, 63 and 255 others
    with seeded lengths in [1, 32768], at random slots.  The batches take every
    scheduling path of bi_attn_decode (one wavefront per chunk; the work queue
    with chunk groups and the merge; whole sequences), and the tracked output
    and lse must be bitwise the same in all of them."""
    hq, n_others = 32, 255
    bt = long_batch
    rng = np.random.default_rng(9)
    for L in (32768, 20001):
        ref = None
        for B in (1, 16, 64, 256):
            others = sorted(rng.choice(np.arange(1, n_others + 1), size=B - 1, replace=False).tolist())
            pos = int(rng.integers(0, B))
            ids = others[:pos] + [0] + others[pos:]
            log_case(f"long-context decode L={L} B={B} slot={pos}")
            idx = torch.tensor(ids, device=DEV)
            lt = bt.lens[idx].clone()
            lt[pos] = L
            out, lse = bi.bi_attn_decode(bt.q[idx].contiguous(), bt.kc, bt.vc, bt.bt[idx].contiguous(), lt, 32768,
                                         bt.scale, lse=torch.empty((B, hq), dtype=torch.float32, device=DEV))
            got = (out[pos].clone(), lse[pos].clone())
            if ref is None:
                ref = got
                ro, rl = O.decode_attention(f64(bt.q[:1]), [f64(bt.kv[0][0][:L])], [f64(bt.kv[0][1][:L])], bt.scale)
                assert_bf16_close(got[0][None], ro, f"long-context L={L}")
                assert_f32_close(got[1][None], rl, f"long-context lse L={L}")
            assert_bitwise(got[0], ref[0], f"tracked output L={L} at B={B} slot={pos}")
            assert_bitwise(got[1], ref[1], f"tracked lse L={L} at B={B} slot={pos}")


def test_decode_long_context_growth_sweep(long_batch):
    """The long-context workload's growth check, sampled at every chunk
    boundary: the tracked request at KV lengths 256k - 1, 256k and 256k + 1 for
    every k up to 32768 (the last chunk one token short of full, full, and a
    new one-token chunk), with a new seeded query at every length.  At each
    length it is decoded alone (max_seq_len = its length) and among 0..255
    others drawn at random from the 255 (max_seq_len 32768), at a random slot;
    output and lse must be bitwise equal.  Sampled lengths against the oracle."""
    bt, hq = long_batch, 32
    rng = np.random.default_rng(12)
    steps = sorted({L for k in range(129) for L in (256 * k - 1, 256 * k, 256 * k + 1) if 1 <= L <= 32768})
    sample = {1, 255, 257, 4097, 16383, 32767, 32768}
    for L in steps:
        q = W.randn_bf16((1, hq, 128), W.SEED_LONG, "q", 20_000 + L, device=DEV)
        lt1 = torch.tensor([L], dtype=torch.int32, device=DEV)
        o1, l1 = bi.bi_attn_decode(q, bt.kc, bt.vc, bt.bt[:1], lt1, L, bt.scale,
                                   lse=torch.empty((1, hq), dtype=torch.float32, device=DEV))
        k = int(rng.integers(0, 256))
        others = rng.choice(np.arange(1, 256), size=k, replace=False).tolist()
        pos = int(rng.integers(0, k + 1))
        ids = others[:pos] + [0] + others[pos:]
        idx = torch.tensor(ids, device=DEV)
        qq = bt.q[idx].clone()
        qq[pos] = q[0]
        lt = bt.lens[idx].clone()
        lt[pos] = L
        o, l = bi.bi_attn_decode(qq, bt.kc, bt.vc, bt.bt[idx].contiguous(), lt, 32768, bt.scale,
                                 lse=torch.empty((k + 1, hq), dtype=torch.float32, device=DEV))
        if L in sample:
            log_case(f"long-context growth L={L} with {k} co-batched at slot {pos}")
            ro, rl = O.decode_attention(f64(q), [f64(bt.kv[0][0][:L])], [f64(bt.kv[0][1][:L])], bt.scale)
            assert_bf16_close(o1, ro, f"growth L={L} vs oracle")
            assert_f32_close(l1, rl, f"growth L={L} lse vs oracle")
        assert_bitwise(o[pos], o1[0], f"tracked output at L={L} with {k} co-batched (slot {pos})")
        assert_bitwise(l[pos], l1[0], f"tracked lse at L={L} with {k} co-batched (slot {pos})")


# ---------------------------------------------------------------- prefill

def _prefill_setup(prefixes, chunk_lens, hq=32, hkv=8, d=128, base=W.SEED_MIXED, perm_index=0):
    """Sequences whose caches already hold prefix + chunk tokens (chunk appended)."""
    total = [p + n for p, n in zip(prefixes, chunk_lens)]
    bt = Batch(range(len(prefixes)), total, hq, hkv, d, base, perm_index=perm_index)
    qs = [W.randn_bf16((n, hq, d), base, "q", 500 + s, device=DEV) for s, n in enumerate(chunk_lens)]
    q = torch.cat(qs).contiguous()
    q_start = torch.tensor([0] + np.cumsum(chunk_lens).tolist(), dtype=torch.int32, device=DEV)
    ctx = torch.tensor(prefixes, dtype=torch.int32, device=DEV)
    return bt, q, q_start, ctx


def _prefill(bt, q, q_start, ctx, max_q_len):
    lse = torch.empty((q.shape[0], bt.hq), dtype=torch.float32, device=DEV)
    return bi.bi_attn_prefill(q, q_start, ctx, max_q_len, bt.kc, bt.vc, bt.bt, bt.scale, lse=lse)


@pytest.mark.parametrize("prefixes,chunks", [([0, 200, 700], [64, 300, 512]), ([5000, 1], [512, 17])])
def test_prefill_parity(prefixes, chunks):
    log_case(f"prefill parity prefixes={prefixes} chunks={chunks}")
    bt, q, q_start, ctx = _prefill_setup(prefixes, chunks)
    out, lse = _prefill(bt, q, q_start, ctx, max(chunks))
    qs = q_start.cpu().tolist()
    for s, (p, n) in enumerate(zip(prefixes, chunks)):
        rows = sorted({0, 1, n // 2, n - 1})
        k, v = f64(bt.kv[s][0]), f64(bt.kv[s][1])
        qq = f64(q[qs[s]:qs[s + 1]])
        for i in rows:
            ro, rl = O.decode_attention(qq[i][None], [k[:p + i + 1]], [v[:p + i + 1]], bt.scale)
            assert_bf16_close(out[qs[s] + i], ro[0], f"seq {s} row {i}")
            assert_f32_close(lse[qs[s] + i], rl[0], f"seq {s} row {i} lse")


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (64, 4, 128), (1, 1, 64)])
def test_prefill_equals_token_by_token_decode(hq, hkv, d):
    prefixes, chunks = [0, 250, 1100], [300, 512, 40]
    log_case(f"prefill == decode hq={hq} hkv={hkv} d={d}")
    bt, q, q_start, ctx = _prefill_setup(prefixes, chunks, hq, hkv, d)
    out, lse = _prefill(bt, q, q_start, ctx, max(chunks))
    qs = q_start.cpu().tolist()
    for s, (p, n) in enumerate(zip(prefixes, chunks)):
        # decode query i of the chunk with seq_len p + i + 1, all as one batch
        lens = torch.arange(p + 1, p + n + 1, dtype=torch.int32, device=DEV)
        btab = bt.bt[s:s + 1].repeat(n, 1).contiguous()
        qd = q[qs[s]:qs[s + 1]].contiguous()
        lsed = torch.empty((n, hq), dtype=torch.float32, device=DEV)
        od, ld = bi.bi_attn_decode(qd, bt.kc, bt.vc, btab, lens, p + n, bt.scale, lse=lsed)
        assert_bitwise(out[qs[s]:qs[s + 1]], od, f"seq {s}: prefill rows vs decode")
        assert_bitwise(lse[qs[s]:qs[s + 1]], ld, f"seq {s}: prefill lse vs decode")
    # and literally one token at a time for the first rows of sequence 1
    s, p = 1, prefixes[1]
    for i in (0, 1, 255, 256):
        od, ld = bi.bi_attn_decode(q[qs[s] + i][None].contiguous(), bt.kc, bt.vc, bt.bt[s:s + 1].contiguous(),
                                   torch.tensor([p + i + 1], dtype=torch.int32, device=DEV), p + i + 1,
                                   bt.scale, lse=torch.empty((1, hq), dtype=torch.float32, device=DEV))
        assert_bitwise(out[qs[s] + i], od[0], f"row {i}: prefill vs single decode")


def _steep_kv(kind):
    """K whose dimension 0 carries a steep score pattern against queries with
    q[0] = 4 (the rest small noise): 'ramp' rises by about 12 log2 units per
    32-key sub-block; 'spikes' puts isolated keys far above everything before
    them, inside and across 256-key chunks."""
    def fn(r, L, hkv, d, base, device="cpu"):
        k, v = W.request_kv(r, L, hkv, d, base, device=device)
        k = k.float() * 0.3
        j = torch.arange(L, device=device, dtype=torch.float32)
        if kind == "ramp":
            k[:, :, 0] = 0.75 * j[:, None]
        else:
            for pos, h in ((5, 40.0), (77, 60.0), (300, 90.0), (301, 95.0), (700, 140.0), (990, 180.0)):
                if pos < L:
                    k[pos, :, 0] += h
        return k.to(torch.bfloat16), v
    return fn


def _assert_weight_rounding_bound(gpu, q, k, v, scale, ref, what):
    """Element-wise form of the attention error bound: with w the exact
    softmax weights (per kv head group, from the oracle's inputs), rounding
    each p to bf16 (unit roundoff 2^-8: 8 significant bits) moves o_d by at
    most 2^-8 sum_j w_j |v_jd|, and the bf16 output adds at most 2^-8 |o_d|
    (a 2 % margin and 1e-6 absolute cover the fp32 sums).  A near-one-hot
    softmax whose few values cancel can exceed a fixed fraction of the row
    RMS while still meeting this bound."""
    hq, hkv = q.shape[0], k.shape[1]
    G = hq // hkv
    g = f64(gpu)
    for h in range(hq):
        kk, vv = k[:, h // G], v[:, h // G]
        sc = scale * (kk @ q[h])
        w = np.exp(sc - sc.max())
        w /= w.sum()
        bound = 1.02 * 2.0 ** -8 * (w @ np.abs(vv) + np.abs(ref[h])) + 1e-6
        err = np.abs(g[h] - ref[h])
        assert np.all(err <= bound), f"{what} head {h}: error {err.max():.3e} above the bound at {int(np.argmax(err - bound))}"


@pytest.mark.parametrize("kind", ["ramp", "spikes"])
def test_lazy_reference_moves(kind):
    """Scores that pass the running reference by far more than the slack, on
    most sub-blocks (ramp) or at isolated keys (spikes), so that every raise of
    the reference with its rescale of l and o, inside a chunk and in the merge
    across chunks, runs: prefill against the oracle on sampled rows and
    bitwise against decode on every row."""
    prefixes, chunks = [0, 250, 700], [300, 512, 300]
    log_case(f"lazy reference moves kind={kind}")
    total = [p + n for p, n in zip(prefixes, chunks)]
    bt = Batch(range(3), total, 32, 8, 128, W.SEED_MIXED, kv_fn=_steep_kv(kind))
    qs_ = []
    for s, n in enumerate(chunks):
        qq = W.randn_bf16((n, 32, 128), W.SEED_MIXED, "q", 700 + s, device=DEV).float() * 0.3
        qq[:, :, 0] = 4.0
        qs_.append(qq.to(torch.bfloat16))
    q = torch.cat(qs_).contiguous()
    q_start = torch.tensor([0] + np.cumsum(chunks).tolist(), dtype=torch.int32, device=DEV)
    ctx = torch.tensor(prefixes, dtype=torch.int32, device=DEV)
    out, lse = _prefill(bt, q, q_start, ctx, max(chunks))
    qs = q_start.cpu().tolist()
    for s, (p, n) in enumerate(zip(prefixes, chunks)):
        lens = torch.arange(p + 1, p + n + 1, dtype=torch.int32, device=DEV)
        btab = bt.bt[s:s + 1].repeat(n, 1).contiguous()
        qd = q[qs[s]:qs[s + 1]].contiguous()
        od, ld = bi.bi_attn_decode(qd, bt.kc, bt.vc, btab, lens, p + n, bt.scale,
                                   lse=torch.empty((n, 32), dtype=torch.float32, device=DEV))
        assert_bitwise(out[qs[s]:qs[s + 1]], od, f"{kind} seq {s}: prefill rows vs decode")
        assert_bitwise(lse[qs[s]:qs[s + 1]], ld, f"{kind} seq {s}: prefill lse vs decode")
        k, v = f64(bt.kv[s][0]), f64(bt.kv[s][1])
        qq = f64(q[qs[s]:qs[s + 1]])
        for i in sorted({0, 40, n // 2, n - 1}):
            ro, rl = O.decode_attention(qq[i][None], [k[:p + i + 1]], [v[:p + i + 1]], bt.scale)
            _assert_weight_rounding_bound(out[qs[s] + i], qq[i], k[:p + i + 1], v[:p + i + 1], bt.scale, ro[0],
                                          f"{kind} seq {s} row {i}")
            assert_f32_close(lse[qs[s] + i], rl[0], f"{kind} seq {s} row {i} lse")


def test_prefill_many_short_sequences():
    """300 short chunks (1..40 new tokens over caches of 0..600): with the
    placement order table (more than 16 sequences) and without it, bitwise the
    same outputs; sampled rows against the oracle and against decode."""
    rng = np.random.default_rng(30)
    S = 300
    prefixes = [int(x) for x in rng.integers(0, 601, S)]
    chunks = [int(x) for x in rng.integers(1, 41, S)]
    bt, q, q_start, ctx = _prefill_setup(prefixes, chunks, perm_index=4)
    log_case(f"prefill many sequences S={S}")
    lse_a = torch.empty((q.shape[0], 32), dtype=torch.float32, device=DEV)
    lse_b = torch.empty((q.shape[0], 32), dtype=torch.float32, device=DEV)
    ws = torch.full((bi.bi_attn_prefill_workspace_bytes(S),), 255, dtype=torch.uint8, device=DEV)
    oa, _ = bi.bi_attn_prefill(q, q_start, ctx, 40, bt.kc, bt.vc, bt.bt, bt.scale, lse=lse_a, workspace=ws)
    ob, _ = bi.bi_attn_prefill(q, q_start, ctx, 40, bt.kc, bt.vc, bt.bt, bt.scale, lse=lse_b, order_table=False)
    assert_bitwise(oa, ob, "order table vs in-kernel ranking")
    assert_bitwise(lse_a, lse_b, "order table vs in-kernel ranking (lse)")
    qs = q_start.cpu().tolist()
    for s_ in (0, 7, 150, S - 1):
        i = chunks[s_] - 1
        row = qs[s_] + i
        L = prefixes[s_] + i + 1
        ro, rl = O.decode_attention(f64(q[row:row + 1]), [f64(bt.kv[s_][0][:L])], [f64(bt.kv[s_][1][:L])], bt.scale)
        assert_bf16_close(oa[row], ro[0], f"sequence {s_} last row vs oracle")
        assert_f32_close(lse_a[row:row + 1], rl, f"sequence {s_} last row lse vs oracle")
        od, _ = bi.bi_attn_decode(q[row:row + 1], bt.kc, bt.vc, bt.bt[s_:s_ + 1],
                                  torch.tensor([L], dtype=torch.int32, device=DEV), L, bt.scale)
        assert_bitwise(oa[row], od[0], f"sequence {s_} last row: prefill vs decode")


def test_prefill_co_batch_invariance():
    prefixes, chunks = [300, 900, 0, 4000], [512, 100, 256, 333]
    bt, q, q_start, ctx = _prefill_setup(prefixes, chunks)
    out, lse = _prefill(bt, q, q_start, ctx, max(chunks))
    qs = q_start.cpu().tolist()
    # sequence 1 alone (request 1's K/V and queries) on a different page permutation
    one_q = q[qs[1]:qs[2]].contiguous()
    one = Batch([1], [prefixes[1] + chunks[1]], 32, 8, 128, W.SEED_MIXED, perm_index=9)
    o1, l1 = bi.bi_attn_prefill(one_q, torch.tensor([0, chunks[1]], dtype=torch.int32, device=DEV),
                                torch.tensor([prefixes[1]], dtype=torch.int32, device=DEV), 512,
                                one.kc, one.vc, one.bt, one.scale,
                                lse=torch.empty((chunks[1], 32), dtype=torch.float32, device=DEV))
    assert_bitwise(out[qs[1]:qs[2]], o1, "sequence 1 prefill alone vs co-batched")
    assert_bitwise(lse[qs[1]:qs[2]], l1, "sequence 1 prefill lse alone vs co-batched")


def test_shared_prefix_pages_are_bitwise_transparent():
    """Prefix caching: requests A and B share the physical pages of a 320-token
    prefix (20 pages, across the first chunk boundary); C holds B's tokens in
    pages of its own.  B and C give bitwise the same decode and prefill
    outputs, and B matches the oracle."""
    hq, hkv, d, ps = 32, 8, 128, 16
    P, la, lb = 320, 150, 400
    npre, na, nb = P // ps, -(-la // ps), -(-lb // ps)
    nc = npre + nb
    pool = npre + na + nb + nc + 3
    perm = torch.randperm(pool, generator=torch.Generator().manual_seed(11)).to(torch.int32)
    pre, pa = perm[:npre], perm[npre:npre + na]
    pb, pc = perm[npre + na:npre + na + nb], perm[npre + na + nb:npre + na + nb + nc]
    pages = [torch.cat([pre, pa]), torch.cat([pre, pb]), pc]
    mp = max(len(x) for x in pages)
    bt = torch.full((3, mp), -1, dtype=torch.int32)
    for i, x in enumerate(pages):
        bt[i, :len(x)] = x
    bt = bt.to(DEV)

    def slots(pg, t0, t1):
        t = torch.arange(t0, t1, dtype=torch.int64)
        return (pg[(t // ps)].to(torch.int64) * ps + t % ps).to(torch.int32)

    kp, vp = W.request_kv(900, P, hkv, d, W.SEED_MIXED, device=DEV)
    ka, va = W.request_kv(901, la, hkv, d, W.SEED_MIXED, device=DEV)
    kb, vb = W.request_kv(902, lb, hkv, d, W.SEED_MIXED, device=DEV)
    kc, vc = bi.alloc_kv_cache(pool, hkv, d, ps, fill=NAN)
    k_all = torch.cat([kp, ka, kb, kp, kb]).contiguous()
    v_all = torch.cat([vp, va, vb, vp, vb]).contiguous()
    sm = torch.cat([slots(pages[0], 0, P), slots(pages[0], P, P + la), slots(pages[1], P, P + lb),
                    slots(pages[2], 0, P + lb)]).to(DEV)
    bi.bi_kv_append(k_all, v_all, sm, kc, vc)

    # decode: B (shared prefix) and C (own pages) with one query, A beside them
    q = W.randn_bf16((3, hq, d), W.SEED_MIXED, "q", 903, device=DEV)
    q[2] = q[1]
    lens = torch.tensor([P + la, P + lb, P + lb], dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    out, lse = bi.bi_attn_decode(q, kc, vc, bt, lens, P + lb, scale,
                                 lse=torch.empty((3, hq), dtype=torch.float32, device=DEV))
    assert_bitwise(out[1], out[2], "decode: shared prefix pages vs own pages")
    assert_bitwise(lse[1], lse[2], "decode lse: shared prefix pages vs own pages")
    ro, rl = O.decode_attention(f64(q[1:2]), [f64(torch.cat([kp, kb]))], [f64(torch.cat([vp, vb]))], scale)
    assert_bf16_close(out[1], ro[0], "decode B vs oracle")
    assert_f32_close(lse[1], rl[0], "decode B lse vs oracle")
    ra, _ = O.decode_attention(f64(q[0:1]), [f64(torch.cat([kp, ka]))], [f64(torch.cat([vp, va]))], scale)
    assert_bf16_close(out[0], ra[0], "decode A vs oracle")

    # prefill: the last 200 tokens of B and of C as the chunk, the same queries
    n = 200
    qp = W.randn_bf16((n, hq, d), W.SEED_MIXED, "q", 904, device=DEV)
    qq = torch.cat([qp, qp]).contiguous()
    q_start = torch.tensor([0, n, 2 * n], dtype=torch.int32, device=DEV)
    ctx = torch.tensor([P + lb - n, P + lb - n], dtype=torch.int32, device=DEV)
    op, lp = bi.bi_attn_prefill(qq, q_start, ctx, n, kc, vc, bt[1:].contiguous(), scale,
                                lse=torch.empty((2 * n, hq), dtype=torch.float32, device=DEV))
    assert_bitwise(op[:n], op[n:], "prefill: shared prefix pages vs own pages")
    assert_bitwise(lp[:n], lp[n:], "prefill lse: shared prefix pages vs own pages")


# ---------------------------------------------------------------- edges and errors

def test_decode_edges():
    bt = Batch(range(3), [5, 300, 17], 32, 8, 128, 21)
    lens = torch.tensor([0, 300, 17], dtype=torch.int32, device=DEV)
    out, lse = bt.decode(lens=lens)
    assert torch.all(out[0].view(torch.int16) == 0)
    assert torch.all(torch.isneginf(lse[0]))
    ref_o, ref_l = bt.decode()
    assert_bitwise(out[1:], ref_o[1:], "other requests unaffected by an empty one")
    # max_seq_len below a length clamps that length (no out-of-range chunk)
    o2, _ = bt.decode(max_seq_len=256, lens=torch.tensor([5, 256, 17], dtype=torch.int32, device=DEV))
    o3, _ = bt.decode(max_seq_len=256, lens=torch.tensor([5, 300, 17], dtype=torch.int32, device=DEV))
    assert_bitwise(o3, o2, "seq_len clamped to max_seq_len")
    # a block table entry outside the pool reads as zeros instead of faulting
    btab = bt.bt.clone()
    btab[1, 3] = 10 ** 6
    o4, _ = bi.bi_attn_decode(bt.q, bt.kc, bt.vc, btab, bt.lens, 300, bt.scale)
    assert torch.isfinite(o4.float()).all()


@pytest.mark.parametrize("B,max_len,msl", [(160, 1400, 1200), (40, 4500, 4000)])
def test_decode_work_queue_edges(B, max_len, msl):
    """Past 2048 (sequence, kv head, chunk) items the decode wavefronts take
    their work from a queue: whole sequences once there are enough (sequence,
    kv head) pairs (160 x 8 here), otherwise groups of chunks whose partials
    the merge kernel folds after the group-0 wavefront's running state (40 x 8
    here, groups of 5 chunks).  Empty sequences, lengths clamped by max_seq_len
    and a workspace full of garbage must give, for every request, bitwise what
    decoding it alone gives (one request: one wavefront per chunk and the merge
    kernel)."""
    lens = [int(x) for x in torch.randint(1, max_len, (B,), generator=torch.Generator().manual_seed(5))]
    bt = Batch(range(B), lens, 32, 8, 128, 23)
    run_lens = list(lens)
    for i in (0, 17, B - 1):
        run_lens[i] = 0
    ws = torch.full((bi.bi_attn_decode_workspace_bytes(B, 32, 128, msl),), 255, dtype=torch.uint8, device=DEV)
    lt = torch.tensor(run_lens, dtype=torch.int32, device=DEV)
    out, lse = bt.decode(max_seq_len=msl, lens=lt, workspace=ws)
    clamped = [i for i in range(B) if run_lens[i] > msl]
    assert clamped, "some lengths exceed max_seq_len"
    longest = sorted(range(B), key=lambda i: -min(run_lens[i], msl))[:3]
    for i in (0, 17, B - 1, 1, 2, B // 2, B - 2, *clamped[:3], *longest):
        log_case(f"decode queue edges B={B} request {i} len {run_lens[i]}")
        o1, l1 = bi.bi_attn_decode(bt.q[i:i + 1], bt.kc, bt.vc, bt.bt[i:i + 1], lt[i:i + 1], msl, bt.scale,
                                   lse=torch.empty((1, 32), dtype=torch.float32, device=DEV))
        assert_bitwise(out[i:i + 1], o1, f"request {i}: queue vs alone")
        assert_bitwise(lse[i:i + 1], l1, f"request {i} lse: queue vs alone")
        if run_lens[i] == 0:
            assert torch.all(out[i].view(torch.int16) == 0) and torch.all(torch.isneginf(lse[i]))
    again, _ = bt.decode(max_seq_len=msl, lens=lt, workspace=ws)
    assert_bitwise(again, out, "queue: repeat with the workspace left by the previous call")
    no_lse, _ = bi.bi_attn_decode(bt.q, bt.kc, bt.vc, bt.bt, lt, msl, bt.scale, lse=None, workspace=ws)
    assert_bitwise(no_lse, out, "queue: no lse output")


@pytest.mark.parametrize("B,hq,hkv,msl", [
    (16, 32, 8, 4096),     # 16 x 8 x 16 = 2048 chunk items: one wavefront per chunk, then the merge kernel
    (17, 32, 8, 4096),     # 2176 items: work queue, chunk groups of 2 + merge
    (2048, 8, 1, 256),     # 2048 items (one chunk each): per-chunk grid
    (2049, 8, 1, 256),     # 2049 items: work queue, whole sequences (one chunk is the whole sequence)
    (127, 32, 8, 1024),    # 1016 (sequence, kv head) pairs: queue with chunk groups + merge
    (128, 32, 8, 1024),    # 1024 pairs: whole-sequence queue, no merge
    (1023, 16, 1, 1024),   # 1023 pairs: chunk groups of 3 + merge
    (1024, 16, 1, 1024)])  # 1024 pairs: whole sequences
def test_decode_dispatch_edges(B, hq, hkv, msl):
    """bi_attn_decode picks its schedule from the batch shape: per-chunk grid
    up to 2048 (sequence, kv head, chunk) items, then a work queue of chunk
    groups, and whole sequences from 1024 (sequence, kv head) pairs on.  The
    arithmetic of a request is the same on every path; at both sides of each
    threshold sampled requests (first, last, longest, random) must equal,
    bit for bit, the request decoded alone."""
    lens = [int(x) for x in torch.randint(1, msl + 1, (B,), generator=torch.Generator().manual_seed(B * 7 + hkv))]
    lens[B // 3] = msl
    bt = Batch(range(B), lens, hq, hkv, 128, 37)
    log_case(f"decode dispatch edge B={B} {hq}/{hkv} max_seq_len={msl}")
    out, lse = bt.decode(max_seq_len=msl)
    picks = sorted({0, B - 1, B // 3, *torch.randint(0, B, (13,), generator=torch.Generator().manual_seed(B)).tolist()})
    for i in picks:
        o1, l1 = bi.bi_attn_decode(bt.q[i:i + 1], bt.kc, bt.vc, bt.bt[i:i + 1], bt.lens[i:i + 1], msl, bt.scale,
                                   lse=torch.empty((1, hq), dtype=torch.float32, device=DEV))
        assert_bitwise(out[i:i + 1], o1, f"request {i} (L={lens[i]}): B={B} vs alone")
        assert_bitwise(lse[i:i + 1], l1, f"request {i} lse: B={B} vs alone")
    ro, rl = bt.oracle([B // 3])
    assert_bf16_close(out[B // 3], ro[0], f"request {B // 3} vs oracle")
    assert_f32_close(lse[B // 3:B // 3 + 1], rl, f"request {B // 3} lse vs oracle")


@pytest.mark.parametrize("B,hq,hkv,d,ps,max_len", [(40, 8, 8, 64, 32, 3000), (300, 16, 1, 128, 256, 2000),
                                                   (130, 64, 4, 128, 64, 4096), (600, 4, 2, 64, 16, 1000)])
def test_decode_queue_geometries(B, hq, hkv, d, ps, max_len):
    """The work-queue paths (whole sequences, chunk groups + merge) across head
    sizes, group sizes 1..16 and page sizes 16..256: every request of the batch
    bitwise equal to decoding it alone (the per-chunk path), and sampled
    requests against the oracle."""
    lens = [int(x) for x in torch.randint(1, max_len + 1, (B,), generator=torch.Generator().manual_seed(B + d))]
    bt = Batch(range(B), lens, hq, hkv, d, 31, page_size=ps)
    log_case(f"decode queue geometry B={B} {hq}/{hkv} D={d} page={ps}")
    out, lse = bt.decode(max_seq_len=max_len)
    for i in range(B):
        o1, l1 = bi.bi_attn_decode(bt.q[i:i + 1], bt.kc, bt.vc, bt.bt[i:i + 1], bt.lens[i:i + 1], max_len, bt.scale,
                                   lse=torch.empty((1, hq), dtype=torch.float32, device=DEV))
        assert_bitwise(out[i:i + 1], o1, f"request {i} (L={lens[i]}): batch vs alone")
        assert_bitwise(lse[i:i + 1], l1, f"request {i} lse: batch vs alone")
    longest = max(range(B), key=lambda i: lens[i])
    for i in (0, longest):
        ro, rl = bt.oracle([i])
        assert_bf16_close(out[i], ro[0], f"request {i} vs oracle")
        assert_f32_close(lse[i:i + 1], rl, f"request {i} lse vs oracle")


def test_attention_errors():
    bt = Batch([0], [10], 32, 8, 128, 22)
    with pytest.raises(bi.BiError) as e:
        bi.bi_attn_decode(bt.q, bt.kc, bt.vc, bt.bt, bt.lens, 10, bt.scale,
                          workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == bi.BI_ERR_WORKSPACE
    q3 = torch.zeros((1, 24, 128), dtype=torch.bfloat16, device=DEV)   # group size 3
    with pytest.raises(bi.BiError) as e:
        bi.bi_attn_decode(q3, bt.kc, bt.vc, bt.bt, bt.lens, 10, bt.scale)
    assert e.value.status in (bi.BI_ERR_UNSUPPORTED, bi.BI_ERR_INVALID_ARG)
    kc, vc = bi.alloc_kv_cache(4, 8, 96, 16)
    with pytest.raises(bi.BiError) as e:
        bi.bi_attn_decode(torch.zeros((1, 32, 96), dtype=torch.bfloat16, device=DEV), kc, vc, bt.bt, bt.lens,
                          10, bt.scale)
    assert e.value.status == bi.BI_ERR_UNSUPPORTED


def test_strided_fused_qkv_inputs():
    # q / k / v read straight out of a fused QKV projection output [B, 6144].
    B, hq, hkv, d = 12, 32, 8, 128
    lens = W.decode_lengths(range(B), 31)
    bt = Batch(range(B), lens, hq, hkv, d, 31)
    qkv = W.randn_bf16((B, 6144), 31, "x", 5, device=DEV)
    q, k, v = (qkv[:, :4096].view(B, hq, d), qkv[:, 4096:5120].view(B, hkv, d), qkv[:, 5120:].view(B, hkv, d))
    o1, _ = bi.bi_attn_decode(q, bt.kc, bt.vc, bt.bt, bt.lens, 4096, bt.scale)
    o2, _ = bi.bi_attn_decode(q.contiguous(), bt.kc, bt.vc, bt.bt, bt.lens, 4096, bt.scale)
    assert_bitwise(o1, o2, "strided q")
    kc2, vc2 = bt.kc.clone(), bt.vc.clone()
    slots = torch.tensor([5, 77, 200, 3, 9, 11, 13, 15, 17, 19, 21, 23], dtype=torch.int32, device=DEV)
    bi.bi_kv_append(k, v, slots, bt.kc, bt.vc)
    bi.bi_kv_append(k.contiguous(), v.contiguous(), slots, kc2, vc2)
    assert_bitwise(bt.kc, kc2, "strided k append")
    assert_bitwise(bt.vc, vc2, "strided v append")


@pytest.mark.parametrize("ps", [32, 256])
def test_page_sizes_decode_parity_and_prefill_equality(ps):
    lens = [1000, 37, 600]
    log_case(f"page size {ps}")
    bt = Batch(range(3), lens, 32, 8, 128, 41, page_size=ps)
    out, lse = bt.decode()
    ro, rl = bt.oracle([0, 1, 2])
    for b in range(3):
        assert_bf16_close(out[b], ro[b], f"ps={ps} request {b}")
    assert_f32_close(lse, rl, f"ps={ps} lse")
    # prefill of the last 64 tokens of request 0 == decode of the same rows
    p, n = 1000 - 64, 64
    q = W.randn_bf16((n, 32, 128), 41, "q", 77, device=DEV)
    po, pl = bi.bi_attn_prefill(q, torch.tensor([0, n], dtype=torch.int32, device=DEV),
                                torch.tensor([p], dtype=torch.int32, device=DEV), n, bt.kc, bt.vc,
                                bt.bt[:1].contiguous(), bt.scale,
                                lse=torch.empty((n, 32), dtype=torch.float32, device=DEV))
    od, ld = bi.bi_attn_decode(q, bt.kc, bt.vc, bt.bt[:1].repeat(n, 1).contiguous(),
                               torch.arange(p + 1, p + n + 1, dtype=torch.int32, device=DEV), 1000, bt.scale,
                               lse=torch.empty((n, 32), dtype=torch.float32, device=DEV))
    assert_bitwise(po, od, f"ps={ps} prefill vs decode")
    assert_bitwise(pl, ld, f"ps={ps} prefill lse vs decode")
