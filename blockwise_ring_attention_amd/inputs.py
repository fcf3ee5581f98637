"""Seeded synthetic inputs for one rank's share of Ring Attention.

This module only draws random numbers and rounds them to the compute dtype. It holds
none of the method's arithmetic (no positions, masks, scores or softmax), so both the
HIP path and the fp64 oracle can take their inputs from it without sharing any code.

Every array is drawn directly in the layout the library consumes:
  q        [B, Hq, Nq, d]
  k_blocks [c, B, Hkv, n, d]   block j = rank j's keys (owner order)
  v_blocks [c, B, Hkv, n, d]
Draw order is Q, K, V, then (where a workload asks for them) the key outlier rows and
their values, all from one ``numpy.random.default_rng(seed)`` stream (PCG64). Values are
drawn in float32, scaled, then rounded to the workload dtype (bf16: round to nearest
even), so the returned float32 arrays hold exactly the values the GPU sees.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "bf16" or "f32"
    batch: int
    hq: int
    hkv: int
    head_dim: int
    seq: int            # total sequence length S over all c ranks
    c: int              # ring size
    rank: int
    causal: bool
    zigzag: bool
    value_scale: float  # Q, K, V ~ N(0, 1) * value_scale
    seed: int
    key_outlier_frac: float = 0.0   # fraction of key rows redrawn per (b, kv head)
    key_outlier_std: float = 0.0
    doc_median: int = 0             # > 0: packed documents, lognormal lengths with this median
    doc_sigma: float = 0.0
    with_lse: bool = True
    notes: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        """Query rows of the rank's share = KV rows per block (S / c)."""
        return self.seq // self.c


# The workloads the method is measured and checked on: the two fp32 parity shapes, the
# 32k and 128k GQA shares, the 64k non-causal share with key outliers, the 128k share
# with packed documents, and the 32k share's shape in fp32 (the fp32 path at a size that
# fills the GPU).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_c3_d8_fp32", "f32", 1, 1, 1, 8, 12, 3, 0, False, False, 1.0, 0,
                 notes="q 4x8, k/v 12x8 split into 3 blocks of 4; the pages' worked example"),
        Workload("mha_d64_s4k_c4_zigzag_fp32", "f32", 1, 1, 1, 64, 4096, 4, 0, True, True, 1.0, 1,
                 notes="rank 0 owns chunks 0 and 7 of 512 tokens"),
        Workload("gqa32x8_d128_s32k_c8_zigzag_bf16", "bf16", 1, 32, 8, 128, 32768, 8, 3, True, True, 0.5, 2,
                 notes="rank 3 owns chunks 3 and 12 of 2048 tokens"),
        Workload("gqa64x8_d128_s128k_c16_zigzag_bf16", "bf16", 1, 64, 8, 128, 131072, 16, 0, True, True, 0.5, 3,
                 notes="rank 0 owns chunks 0 and 31 of 4096 tokens; emits lse"),
        Workload("mha16_b2_d128_s64k_c8_noncausal_outliers_bf16", "bf16", 2, 16, 16, 128, 65536, 8, 0, False, False,
                 1.0, 4, key_outlier_frac=0.01, key_outlier_std=3.0,
                 notes="1% of key rows per (b, head) redrawn from N(0, 3^2)"),
        Workload("gqa64x8_d128_s128k_c16_zigzag_docs_bf16", "bf16", 1, 64, 8, 128, 131072, 16, 0, True, True, 0.5, 3,
                 doc_median=8192, doc_sigma=1.0,
                 notes="the 128k share with a packed-document mask: lognormal document lengths, median 8192"),
        Workload("gqa32x8_d128_s32k_c8_zigzag_fp32", "f32", 1, 32, 8, 128, 32768, 8, 3, True, True, 0.5, 5,
                 notes="the 32k share's shape in fp32"),
    ]
}


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the workload dtype and return them as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def make_inputs(w: Workload, seed: int | None = None, rows: int | None = None):
    """Draw (q, k_blocks, v_blocks) for workload ``w`` as float32 numpy arrays whose
    values are exactly representable in ``w.dtype``. ``rows`` overrides S / c (for
    scaled-down copies of a workload); ``seed`` overrides ``w.seed``."""
    n = w.rows if rows is None else rows
    rng = np.random.default_rng(w.seed if seed is None else seed)
    s = np.float32(w.value_scale)
    q = rng.standard_normal((w.batch, w.hq, n, w.head_dim), dtype=np.float32) * s
    k = rng.standard_normal((w.c, w.batch, w.hkv, n, w.head_dim), dtype=np.float32) * s
    v = rng.standard_normal((w.c, w.batch, w.hkv, n, w.head_dim), dtype=np.float32) * s
    if w.key_outlier_frac > 0:
        total = w.c * n
        count = int(round(w.key_outlier_frac * total))
        for b in range(w.batch):
            for g in range(w.hkv):
                idx = rng.choice(total, size=count, replace=False)
                vals = rng.standard_normal((count, w.head_dim), dtype=np.float32) * np.float32(w.key_outlier_std)
                k[idx // n, b, g, idx % n] = vals
    return round_to_dtype(q, w.dtype), round_to_dtype(k, w.dtype), round_to_dtype(v, w.dtype)


def doc_start_from_lengths(lengths) -> np.ndarray:
    """The doc_start array of a packed sequence whose documents have ``lengths`` tokens,
    in order: entry p is the position where p's document begins (int32)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if np.any(lengths < 1):
        raise ValueError("document lengths must be positive")
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    return np.repeat(starts, lengths).astype(np.int32)


def draw_document_lengths(total: int, median: float, sigma: float, seed) -> np.ndarray:
    """Seeded lognormal document lengths (at least 1 token) packed into ``total`` tokens;
    the last document is cut to fit."""
    rng = np.random.default_rng(seed)
    lengths = []
    used = 0
    while used < total:
        n = max(1, int(round(float(rng.lognormal(np.log(median), sigma)))))
        n = min(n, total - used)
        lengths.append(n)
        used += n
    return np.asarray(lengths, dtype=np.int64)


def make_doc_start(w: Workload, rows: int | None = None):
    """The workload's document layout as a doc_start array over all c * n positions, or
    None when it has no document mask. Drawn from its own stream (seed, 1), so Q/K/V stay
    those of the same workload without documents."""
    if w.doc_median <= 0:
        return None
    n = w.rows if rows is None else rows
    return doc_start_from_lengths(draw_document_lengths(w.c * n, w.doc_median, w.doc_sigma, [w.seed, 1]))


def random_array(shape, dtype: str, seed: int, scale: float = 1.0) -> np.ndarray:
    """One seeded N(0, scale^2) array rounded to ``dtype`` (for tests of odd shapes)."""
    rng = np.random.default_rng(seed)
    return round_to_dtype(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale), dtype)
