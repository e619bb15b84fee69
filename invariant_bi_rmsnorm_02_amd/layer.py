"""A pre-norm decoder layer (Qwen3-style shapes) composed from the library's
entry points.  Every step is one C-ABI call on the caller's stream; this module
only sequences them and slices views (q, k and v are read straight out of the
fused QKV projection, the gate and up halves out of the fused gate/up one).

    h  = rmsnorm(x, g1)                        bi_rmsnorm
    qkv = h W_qkv^T                            bi_gemm
    cache <- k, v                              bi_kv_append
    a  = attention(q, cache)                   bi_attn_decode / bi_attn_prefill
    r  = x + a W_o^T                           bi_gemm_add
    h2 = rmsnorm(r, g2)                        bi_rmsnorm
    y  = r + (silu(gate) * up) W_down^T        bi_gemm_silu_mul, bi_gemm_add

The residual adds and the gated activation run in the epilogues of the GEMMs
before them (bi_gemm_add, bi_gemm_silu_mul on the gate/up weight with its
rows interleaved).  Each fused call gives bit for bit what the unfused pair
(bi_gemm then bi_add / bi_silu_mul) gives; a `trace` call runs the unfused
steps so that every intermediate can be checked.

Each step is batch-invariant on its own (row-wise reductions in a fixed order,
one GEMM tile and K order, fixed 256-token KV chunks, pointwise work), so a
token's output does not depend on the batch it is computed in, nor on whether
it is prefilled or decoded.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import (bi_add, bi_attn_decode, bi_attn_decode_workspace_bytes, bi_attn_prefill, bi_gemm, bi_gemm_add,
               bi_gemm_silu_mul, bi_kv_append, bi_lm_head_greedy, bi_lm_head_logprobs, bi_moe_ffn, bi_moe_route,
               bi_rmsnorm, bi_silu_mul, interleave_gate_up)


class DecoderLayer:
    """Weights (bf16, on the device): w_qkv [(Hq + 2 Hkv) D, H], w_o [H, Hq D],
    w_gu [2 F, H] (gate rows first, then up), w_down [H, F]; g1, g2 [H].  The
    layer keeps w_gu only as its row-interleaved copy (w_gu_il), the layout of
    bi_gemm_silu_mul; the w_gu property gives the [gate; up] layout back."""

    def __init__(self, w_qkv: torch.Tensor, w_o: torch.Tensor, w_gu: torch.Tensor, w_down: torch.Tensor,
                 g1: torch.Tensor, g2: torch.Tensor, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 eps: float = 1e-6):
        self.w_qkv, self.w_o, self.w_down, self.g1, self.g2 = w_qkv, w_o, w_down, g1, g2
        self.hq, self.hkv, self.d, self.eps = num_q_heads, num_kv_heads, head_dim, eps
        self.scale = 1.0 / math.sqrt(head_dim)
        hd = (num_q_heads + 2 * num_kv_heads) * head_dim
        if w_qkv.shape[0] != hd or w_o.shape != (w_qkv.shape[1], num_q_heads * head_dim):
            raise ValueError("w_qkv / w_o shapes do not match the head layout")
        if w_gu.shape[0] % 2 or w_down.shape != (w_qkv.shape[1], w_gu.shape[0] // 2):
            raise ValueError("w_gu / w_down shapes")
        self.w_gu_il = interleave_gate_up(w_gu)

    @property
    def w_gu(self) -> torch.Tensor:
        """The gate/up weight in its [gate; up] layout (a copy)."""
        f = self.w_gu_il.shape[0] // 2
        return self.w_gu_il.view(f, 2, -1).transpose(0, 1).reshape(2 * f, -1)

    # The three reductions of the layer, one library call each.
    def _norm(self, x: torch.Tensor, gamma: torch.Tensor) -> torch.Tensor:
        return bi_rmsnorm(x, gamma, self.eps)

    def _gemm(self, a: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
        return bi_gemm(a, w)

    def _attend(self, q, k_cache, v_cache, block_table, seq_lens, max_seq_len, workspace):
        if workspace is None:
            need = bi_attn_decode_workspace_bytes(q.shape[0], self.hq, self.d, max_seq_len)
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        return bi_attn_decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, self.scale,
                              workspace=workspace)[0]

    def _qkv(self, x: torch.Tensor, trace: Optional[dict]):
        T = x.shape[0]
        h = self._norm(x, self.g1)
        qkv = self._gemm(h, self.w_qkv)
        if trace is not None:
            trace.update(h=h, qkv=qkv)
        a, b = self.hq * self.d, (self.hq + self.hkv) * self.d
        q = qkv[:, :a].view(T, self.hq, self.d)
        k = qkv[:, a:b].view(T, self.hkv, self.d)
        v = qkv[:, b:].view(T, self.hkv, self.d)
        return q, k, v

    def _tail(self, x: torch.Tensor, attn: torch.Tensor, trace: Optional[dict]) -> torch.Tensor:
        T = x.shape[0]
        a2 = attn.view(T, self.hq * self.d)
        if trace is None:
            r = bi_gemm_add(a2, self.w_o, x)
            h2 = self._norm(r, self.g2)
            m = bi_gemm_silu_mul(h2, self.w_gu_il)
            return bi_gemm_add(m, self.w_down, r, out=r)
        c = self._gemm(a2, self.w_o)
        r = bi_add(x, c)
        h2 = self._norm(r, self.g2)
        gu = self._gemm(h2, self.w_gu_il)                  # columns gate 0, up 0, gate 1, up 1, ...
        gu = torch.cat((gu[:, 0::2], gu[:, 1::2]), dim=1)   # [gate | up]
        m = bi_silu_mul(gu)
        d = self._gemm(m, self.w_down)
        trace.update(attn=attn, c=c, r=r.clone(), h2=h2, gu=gu, m=m, d=d)   # r is overwritten below
        return bi_add(r, d, out=r)

    def decode(self, x: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor, slot_mapping: torch.Tensor, max_seq_len: int,
               workspace: Optional[torch.Tensor] = None, trace: Optional[dict] = None) -> torch.Tensor:
        """x [B, H]: the newest token of each of B sequences; seq_lens count it;
        slot_mapping [B] is where its K/V goes.  Returns y [B, H].  A `trace`
        dict receives every step's output tensor (h, qkv, attn, c, r, h2, gu,
        m, d), for checking the steps one by one; it changes no call."""
        q, k, v = self._qkv(x, trace)
        bi_kv_append(k, v, slot_mapping, k_cache, v_cache)
        attn = self._attend(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, workspace)
        return self._tail(x, attn, trace)

    def prefill(self, x: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                q_start: torch.Tensor, ctx_lens: torch.Tensor, slot_mapping: torch.Tensor,
                max_q_len: int, trace: Optional[dict] = None) -> torch.Tensor:
        """x [T, H]: the new tokens of S sequences back to back (sequence s at
        rows q_start[s] .. q_start[s+1]-1, positions ctx_lens[s] ...);
        slot_mapping [T].  Returns y [T, H].  `trace` as in decode."""
        q, k, v = self._qkv(x, trace)
        bi_kv_append(k, v, slot_mapping, k_cache, v_cache)
        attn, _ = bi_attn_prefill(q, q_start, ctx_lens, max_q_len, k_cache, v_cache, block_table, self.scale)
        return self._tail(x, attn, trace)


class MoEDecoderLayer(DecoderLayer):
    """The same layer with a routed mixture-of-experts MLP (Qwen3-235B-A22B
    shapes: 64/4 heads, 128 experts, top 8, expert FFN 4096 -> 1536 -> 4096):

        h2 = rmsnorm(r, g2)
        ids, w = route(h2 W_gate^T, top_k)     bi_moe_route
        y  = r + sum_s w_s FFN_{ids_s}(h2)     bi_moe_ffn, bi_add

    w_gate [E, H]; w_up [E, F, H]; w_down [E, H, F] (bf16).  The router picks
    a token's experts from that token's fp32 logits alone (larger logit, then
    lower id) and the experts' sum runs in slot order, so the whole layer stays
    batch-invariant."""

    def __init__(self, w_qkv: torch.Tensor, w_o: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                 w_down: torch.Tensor, g1: torch.Tensor, g2: torch.Tensor, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, top_k: int, eps: float = 1e-6):
        self.w_qkv, self.w_o, self.g1, self.g2 = w_qkv, w_o, g1, g2
        self.w_gate, self.w_up, self.w_down_e, self.top_k = w_gate, w_up, w_down, top_k
        self.hq, self.hkv, self.d, self.eps = num_q_heads, num_kv_heads, head_dim, eps
        self.scale = 1.0 / math.sqrt(head_dim)
        hd = (num_q_heads + 2 * num_kv_heads) * head_dim
        H = w_qkv.shape[1]
        if w_qkv.shape[0] != hd or w_o.shape != (H, num_q_heads * head_dim):
            raise ValueError("w_qkv / w_o shapes do not match the head layout")
        E = w_gate.shape[0]
        if w_gate.shape != (E, H) or w_up.dim() != 3 or w_up.shape[0] != E or w_up.shape[2] != H \
                or w_down.shape != (E, H, w_up.shape[1]):
            raise ValueError("w_gate / w_up / w_down shapes")

    def _tail(self, x: torch.Tensor, attn: torch.Tensor, trace: Optional[dict]) -> torch.Tensor:
        T = x.shape[0]
        a2 = attn.view(T, self.hq * self.d)
        if trace is None:
            r = bi_gemm_add(a2, self.w_o, x)
        else:
            c = self._gemm(a2, self.w_o)
            r = bi_add(x, c)
        h2 = self._norm(r, self.g2)
        ids, wts, logits = bi_moe_route(h2, self.w_gate, self.top_k)
        e = bi_moe_ffn(h2, ids, wts, self.w_up, self.w_down_e)
        if trace is not None:   # r is overwritten by the last add below
            trace.update(attn=attn, c=c, r=r.clone(), h2=h2, ids=ids, wts=wts, logits=logits, e=e)
        return bi_add(r, e, out=r)


class LMHead:
    """Final RMSNorm and the vocabulary projection: per token, fp32 logprobs
    (bi_lm_head_logprobs, log_softmax fused into the GEMM) or the greedy token
    and its logprob (bi_lm_head_greedy)."""

    def __init__(self, gamma: torch.Tensor, w: torch.Tensor, eps: float = 1e-6):
        self.gamma, self.w, self.eps = gamma, w, eps

    def logprobs(self, y: torch.Tensor, trace: Optional[dict] = None) -> torch.Tensor:
        hf = bi_rmsnorm(y, self.gamma, self.eps)
        if trace is not None:
            trace["hf"] = hf
        return bi_lm_head_logprobs(hf, self.w)

    def greedy(self, y: torch.Tensor):
        """(token [T] int32, its logprob [T] fp32)."""
        lp = torch.empty((y.shape[0],), dtype=torch.float32, device=y.device)
        return bi_lm_head_greedy(bi_rmsnorm(y, self.gamma, self.eps), self.w, logprob=lp)
