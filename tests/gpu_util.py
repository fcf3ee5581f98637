"""Helpers shared by the GPU parity tests (test code only)."""

from __future__ import annotations

import sys

import numpy as np

# Tolerances of the method's parity bar, against the fp64 oracle.
BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX = 2e-2, 2e-3, 1e-5, 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def run_gpu(q, k, v, c, rank, causal, zigzag, t0=0, t1=None, dtype="bf16", with_lse=True):
    """Upload, run ra.rank_forward, return (out fp64 numpy, lse fp64 numpy or None)."""
    import torch
    import blockwise_ring_attention_amd as ra
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out, lse = ra.rank_forward(qd, kd, vd, c, rank, causal, zigzag, t0, t1, with_lse=with_lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64) if lse is not None else None
    return o, l


def assert_parity(out, ref_out, lse, ref_lse, dtype: str, label: str = ""):
    """The parity bar: bf16 max abs <= 2e-2 and mean abs <= 2e-3; fp32 max abs <= 1e-5;
    lse max abs <= 1e-3 over finite entries, and -inf exactly where the oracle has it."""
    err = np.abs(out - ref_out)
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    if dtype == "bf16":
        assert err.max() <= BF16_MAX, f"{label}: max abs {err.max():.3e}"
        assert err.mean() <= BF16_MEAN, f"{label}: mean abs {err.mean():.3e}"
    else:
        assert err.max() <= F32_MAX, f"{label}: max abs {err.max():.3e}"
    if lse is not None:
        inf_ref = np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(lse), inf_ref), f"{label}: -inf pattern of lse differs"
        if (~inf_ref).any():
            le = np.abs(lse[~inf_ref] - ref_lse[~inf_ref]).max()
            assert le <= LSE_MAX, f"{label}: lse max abs {le:.3e}"
    return float(err.max()), float(err.mean())


def rel_l2(a, b) -> float:
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))
