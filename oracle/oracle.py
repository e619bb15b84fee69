"""Plain, slow, fp64 CPU oracle for the batch-invariant forward-pass kernels.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (no headers, kernels, helpers or constants) and imports
nothing from the product package; the product path never calls it.

Sources (web pages; no code was available):
  [TML]  "Thinking Machines Lab - Defeating Nondeterminism in LLM Inference: The
         Core Role of Batch Invariance" (jasonandjarvis.org summary of the Thinking
         Machines Lab post).  Sections "1. Batch-Invariant RMSNorm",
         "2. Batch-Invariant Matrix Multiplication", "3. Batch-Invariant Attention".
  [BINR] "Batch Invariance and Numerical Reproducibility" (praveentn.live), the
         answer on fixed-size chunks (1,000-token cache example) and the answer on
         sampler/trainer logprob agreement.
  [HADA] "Como superar a não determinismo na inferência de LLMs" (pt.news.hada.io),
         section "Projeto de kernels invariantes a batch ...", Attention bullets.

Every method on those pages is a re-ordering (data-parallel rows, 2-D output
tiles, fixed-size split-KV with a log-sum-exp merge) that reaches, in exact
arithmetic, the plain mathematical definition of the operation.  So the oracle
computes the *definitions*, in float64, from the same bf16 input bits the GPU
reads.  Where the pages leave a step open, the reading taken is stated at the
function.

Pins (what fixes this code to something other than itself) live in
``tests/test_oracle.py``: closed forms, brute force in exact rational/integer
arithmetic on tiny inputs, invariants, and the pages' worked example
(``tests/golden/chunk_example.json``).  Every function below is pinned; none is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

# Fixed split size of the split-KV reduction ([BINR] fixed-size chunks answer:
# a 1,000-token cache becomes three 256-token chunks plus one of 232).
KV_CHUNK = 256


# ---------------------------------------------------------------------------
# bfloat16 <-> float64 (exact decode; round-to-nearest-even encode)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (any 16-bit integer dtype) to float64, exactly.

    A bfloat16 is the upper half of an IEEE binary32, so the value is the float32
    whose bits are ``bits << 16``.
    """
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), return uint16 bits.

    Rounds once, directly from float64 (no intermediate float32 step).  bfloat16
    keeps 8 significant bits and the float32 exponent range: normal numbers have
    a quantum of 2**(e-8) for x = f * 2**e with 0.5 <= |f| < 1, and subnormals a
    fixed quantum of 2**-133.  Overflow goes to +-inf; NaN maps to a quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = x[finite]
    _, e = np.frexp(xf)
    q = np.maximum(e, -125) - 8                      # exponent of the quantum
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)       # np.rint rounds half to even
    out[finite] = r
    out[~finite] = x[~finite]
    big = np.abs(out) > float(np.finfo(np.float32).max)
    out[big] = np.copysign(np.inf, out[big])         # overflow rounds to +-inf
    f32 = out.astype(np.float32)                     # exact: every finite r has an 8-bit significand
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(x)] = np.uint16(0x7FC0)
    return bits


# ---------------------------------------------------------------------------
# RMSNorm  ([TML] "1. Batch-Invariant RMSNorm")
# ---------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation of every row of ``x`` [R, H].

    The page names the operation (root mean square normalisation, one reduction
    per batch element) but prints no formula.  Reading taken: the standard form
    with eps inside the root and the gain applied as is (not 1 + gamma):
        y[r, j] = x[r, j] / sqrt(mean_j x[r, j]**2 + eps) * gamma[j].
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * g


# ---------------------------------------------------------------------------
# GEMM  ([TML] "2. Batch-Invariant Matrix Multiplication")
# ---------------------------------------------------------------------------

def gemm(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """C = A @ W^T with A [M, K] (activations) and W [N, K] (weights stored as
    [out_features, in_features]), in float64.  The page's tiled data-parallel
    matmul computes exactly this product; the library primitive is the step.
    """
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return a @ w.T


# ---------------------------------------------------------------------------
# Attention  ([TML] "3. Batch-Invariant Attention"; [BINR] fixed-size chunks)
# ---------------------------------------------------------------------------

def kv_chunks(length: int, chunk: int = KV_CHUNK) -> List[int]:
    """Sizes of the fixed-size split-KV chunks of a cache of ``length`` tokens.

    Chunks are anchored at position 0 and only the last one may be partial, so
    the decomposition of a prefix never changes as the cache grows.
    """
    if length < 0:
        raise ValueError("negative length")
    full, rest = divmod(int(length), int(chunk))
    return [chunk] * full + ([rest] if rest else [])


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query mapping (reading: consecutive groups, as in Qwen3):
    q head h reads kv head h // (Hq / Hkv)."""
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return q_head // (num_q_heads // num_kv_heads)


def attention_row(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                  scale: float) -> Tuple[np.ndarray, float]:
    """Softmax attention of one query vector q [D] over L keys/values [L, D].

    s_j = scale * <q, k_j>;  o = sum_j softmax(s)_j v_j;  lse = log sum_j exp(s_j).
    Returns (o [D], lse).  The max is subtracted before exponentiation only to
    stay in range; in exact arithmetic it cancels.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    if k.shape[0] == 0:
        raise ValueError("attention over an empty key set is undefined")
    s = float(scale) * (k @ q)
    m = np.max(s)
    p = np.exp(s - m)
    l = np.sum(p)
    return (p @ v) / l, float(m + np.log(l))


def decode_attention(q: np.ndarray, k_seqs: Sequence[np.ndarray], v_seqs: Sequence[np.ndarray],
                     scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention for B requests, one query token each.

    q [B, Hq, D]; k_seqs[b], v_seqs[b] are request b's *logical* cache
    [L_b, Hkv, D] (contiguous, no paging: the oracle never sees page tables).
    Returns out [B, Hq, D] and lse [B, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        kb = np.asarray(k_seqs[b], dtype=np.float64)
        vb = np.asarray(v_seqs[b], dtype=np.float64)
        Hkv = kb.shape[1]
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[b, h], lse[b, h] = attention_row(q[b, h], kb[:, g, :], vb[:, g, :], scale)
    return out, lse


def prefill_attention(q: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray, ctx_len: int,
                      scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Causal attention for one chunk of n new tokens of a sequence (chunked prefill).

    q [n, Hq, D] are the chunk's queries; k_seq, v_seq [ctx_len + n, Hkv, D] hold
    the cached prefix followed by the chunk's own keys/values (one layout for
    cached and new tokens: [HADA] Attention bullets, [TML] "FlashAttention with
    KV Cache").  Reading of the mask (pages silent): the query at absolute
    position p = ctx_len + i attends keys 0..p inclusive.
    """
    q = np.asarray(q, dtype=np.float64)
    n, Hq, D = q.shape
    k = np.asarray(k_seq, dtype=np.float64)
    v = np.asarray(v_seq, dtype=np.float64)
    Hkv = k.shape[1]
    if k.shape[0] < ctx_len + n:
        raise ValueError("cache shorter than ctx_len + n")
    out = np.zeros((n, Hq, D))
    lse = np.zeros((n, Hq))
    for i in range(n):
        L = ctx_len + i + 1
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[i, h], lse[i, h] = attention_row(q[i, h], k[:L, g, :], v[:L, g, :], scale)
    return out, lse


def chunk_partial(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                  scale: float) -> Tuple[float, float, np.ndarray]:
    """Un-normalised softmax statistics of one split-KV chunk, in float64:
    m = max_j s_j,  l = sum_j exp(s_j - m),  acc = sum_j exp(s_j - m) v_j."""
    s = float(scale) * (np.asarray(keys, dtype=np.float64) @ np.asarray(q, dtype=np.float64))
    m = float(np.max(s))
    p = np.exp(s - m)
    return m, float(np.sum(p)), p @ np.asarray(values, dtype=np.float64)


def merge_partials(parts: Sequence[Tuple[float, float, np.ndarray]]) -> Tuple[np.ndarray, float]:
    """Fixed-order log-sum-exp merge of chunk partials ([TML] fig. "Fixed Size Split
    KV Strategy"; the merge order is not stated, reading: an ascending left fold
    starting from (m=-inf, l=0, acc=0)).  Returns (o, lse)."""
    m, l, acc = -math.inf, 0.0, None
    for mc, lc, accc in parts:
        mn = max(m, mc)
        alpha = math.exp(m - mn) if m != -math.inf else 0.0
        beta = math.exp(mc - mn)
        l = l * alpha + lc * beta
        acc = accc * beta if acc is None else acc * alpha + accc * beta
        m = mn
    return acc / l, m + math.log(l)


def chunked_attention_row(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                          chunk: int = KV_CHUNK) -> Tuple[np.ndarray, float]:
    """The pages' split-KV method, in float64: fixed-size chunks, per-chunk partial
    statistics, then the ascending merge.  Equal to ``attention_row`` in exact
    arithmetic; used to check that identity and the chunk decomposition."""
    parts = []
    start = 0
    for size in kv_chunks(keys.shape[0], chunk):
        parts.append(chunk_partial(q, keys[start:start + size], values[start:start + size], scale))
        start += size
    return merge_partials(parts)


# ---------------------------------------------------------------------------
# log_softmax ([BINR] answer on sampler/trainer logprob agreement)
# ---------------------------------------------------------------------------

def log_softmax(z: np.ndarray) -> np.ndarray:
    """Row-wise log-probabilities: lp_j = z_j - (max z + log sum_j exp(z_j - max z))."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    return z - (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))


# ---------------------------------------------------------------------------
# Mixture-of-experts combine (workload support; not on the pages)
# ---------------------------------------------------------------------------

def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x / (1 + exp(-x)) (reading of the unstated expert activation)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def moe_ffn(x: np.ndarray, experts: np.ndarray, weights: np.ndarray,
            w_up: Sequence[np.ndarray], w_down: Sequence[np.ndarray]) -> np.ndarray:
    """y_t = sum_s weights[t, s] * W_down[e] @ silu(W_up[e] @ x_t),  e = experts[t, s].

    x [T, H]; experts, weights [T, k]; w_up[e] [F, H]; w_down[e] [H, F].
    Reading (routing and activation are not on the pages): a gate-less SiLU FFN
    per expert and a weighted sum over the k routed slots.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    y = np.zeros((T, H))
    for t in range(T):
        for s in range(experts.shape[1]):
            e = int(experts[t, s])
            h = silu(np.asarray(w_up[e], dtype=np.float64) @ x[t])
            y[t] += float(weights[t, s]) * (np.asarray(w_down[e], dtype=np.float64) @ h)
    return y


def moe_route(x: np.ndarray, w_gate: np.ndarray, top_k: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Token routing of a mixture-of-experts layer (workload support: the
    Qwen3-235B-A22B-shaped layer; routing is not on the pages).

    logits = x @ w_gate^T (x [T, H], w_gate [E, H]); every token takes the
    top_k experts of largest logit, a larger logit first and, among equal
    logits, the lower expert index first (reading: a fixed tie-break, so the
    choice is a function of the token's logits alone); the weights are the
    softmax of the chosen logits, i.e. the softmax over all experts restricted
    to the chosen ones and renormalised.  Returns (experts [T, top_k] int64,
    weights [T, top_k], logits [T, E]).
    """
    logits = gemm(x, w_gate)
    T, E = logits.shape
    experts = np.zeros((T, top_k), dtype=np.int64)
    weights = np.zeros((T, top_k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:top_k]
        experts[t] = order
        z = logits[t, order]
        p = np.exp(z - z.max())
        weights[t] = p / p.sum()
    return experts, weights, logits


# ---------------------------------------------------------------------------
# One decoder layer (workload support; the pages describe no layer)
# ---------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest bfloat16 (ties to even), returned as float64."""
    return bf16_to_f64(f64_to_bf16_bits(x))


def silu_mul(gate_up: np.ndarray) -> np.ndarray:
    """silu(g) * u for rows of a fused gate/up projection [.., 2F]: g is the first
    F columns, u the last F.  Reading (no layer is on the pages): the gated MLP
    of a Qwen3-style decoder layer, down(silu(gate(h)) * up(h))."""
    gu = np.asarray(gate_up, dtype=np.float64)
    f = gu.shape[-1] // 2
    return silu(gu[..., :f]) * gu[..., f:]


def decoder_layer(x: np.ndarray, k_prefix: np.ndarray, v_prefix: np.ndarray, weights: dict,
                  num_q_heads: int, num_kv_heads: int, head_dim: int, eps: float,
                  scale: float, steps: dict = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One pre-norm decoder layer over the T new tokens x [T, H] of one sequence
    whose cache already holds P tokens (k_prefix, v_prefix [P, Hkv, D]).

    Reading (no layer is on the pages): the step sequence of a Qwen3-style layer,
        h = rmsnorm(x, g1); q, k, v = h W_qkv^T; a = causal attention of q over
        the prefix and the new k, v; r = x + a W_o^T; h2 = rmsnorm(r, g2);
        y = r + (silu(h2 W_gate^T) * h2 W_up^T) W_down^T
    with W_gu = [W_gate; W_up] stacked along the output dimension.  The layer's
    activations are bfloat16 tensors, so every step's output is rounded to
    bfloat16 (ties to even) before the next step reads it; each step itself is
    the float64 definition above.  Returns y [T, H] and the new k, v [T, Hkv, D].
    A ``steps`` dict, if given, receives every step's rounded output (h, qkv,
    a, c = a W_o^T, r, h2, gu, m, d = m W_down^T) for error propagation checks.
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    P = np.asarray(k_prefix).shape[0]
    hq, hkv, d = num_q_heads, num_kv_heads, head_dim
    h = round_bf16(rmsnorm(x, weights["g1"], eps))
    qkv = round_bf16(gemm(h, weights["w_qkv"]))
    q = qkv[:, :hq * d].reshape(T, hq, d)
    k = qkv[:, hq * d:(hq + hkv) * d].reshape(T, hkv, d)
    v = qkv[:, (hq + hkv) * d:].reshape(T, hkv, d)
    K = np.concatenate([np.asarray(k_prefix, dtype=np.float64).reshape(P, hkv, d), k])
    V = np.concatenate([np.asarray(v_prefix, dtype=np.float64).reshape(P, hkv, d), v])
    a = round_bf16(prefill_attention(q, K, V, P, scale)[0]).reshape(T, hq * d)
    c = round_bf16(gemm(a, weights["w_o"]))
    r = round_bf16(x + c)
    h2 = round_bf16(rmsnorm(r, weights["g2"], eps))
    gu = round_bf16(gemm(h2, weights["w_gu"]))
    m = round_bf16(silu_mul(gu))
    dn = round_bf16(gemm(m, weights["w_down"]))
    y = round_bf16(r + dn)
    if steps is not None:
        steps.update(h=h, qkv=qkv, a=a, c=c, r=r, h2=h2, gu=gu, m=m, d=dn)
    return y, k, v
