"""Shared test helpers: library loading, bf16 <-> oracle conversion, tolerances.

Tolerances (stated by the workload targets, applied literally):
  bf16 outputs: max relative error <= 1e-2, where the error of element i of a
    row r is |g_i - o_i| / max(|o_i|, rms(o)) with rms over the compared row
    (GEMM/RMSNorm row, attention (request, head) vector).  Elements that
    cancel to near zero are judged against the row's scale instead of their
    own, which a plain relative error would make meaningless.
  fp32 logits / logprobs / lse: max absolute error <= 1e-3.
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import invariant_bi_rmsnorm_02_amd as bi  # noqa: E402
from oracle import oracle as O  # noqa: E402

BF16_REL_TOL = 1e-2
F32_ABS_TOL = 1e-3


def ensure_lib():
    if not os.path.exists(bi.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return bi.lib()


def log_case(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 view of a bf16 or fp32 tensor's values (via the oracle's decoder for bf16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return O.bf16_to_f64(t.contiguous().view(torch.int16).numpy())
    return t.to(torch.float64).numpy()


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view for bitwise comparison."""
    t = t.detach().contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def assert_bitwise(a: torch.Tensor, b: torch.Tensor, what: str) -> None:
    ba, bb = bits(a), bits(b)
    if not torch.equal(ba, bb):
        n = int((ba != bb).sum().item())
        raise AssertionError(f"{what}: {n} of {ba.numel()} elements differ bitwise")


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r_row)), rows along the last axis."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    den = np.maximum(np.abs(r), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - r) / den)) if g.size else 0.0


def assert_bf16_close(gpu: torch.Tensor, ref: np.ndarray, what: str, tol: float = BF16_REL_TOL) -> float:
    err = row_rel_err(f64(gpu), ref)
    assert np.isfinite(err) and err <= tol, f"{what}: max rel err {err:.3e} > {tol}"
    return err


def assert_f32_close(gpu: torch.Tensor, ref: np.ndarray, what: str, tol: float = F32_ABS_TOL) -> float:
    g = f64(gpu)
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    assert np.isfinite(err) and err <= tol, f"{what}: max abs err {err:.3e} > {tol}"
    return err
