"""Blockwise attention assembled from per-block partial results, fp64: a second
implementation used only to pin the full-row oracle (``attention.rank_forward``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it relies on is the fact the pages state, not their update rule: attention over a
row split into key blocks can be rebuilt exactly from what each block gives on its own
("Ring Attention and Ulysses shard a sequence two different ways, ...", section "Ring
Attention: point-to-point rotation, and an online softmax that never sees the whole row
at once"; "What do you do about long sequences and sparse models?", section "How does
attention survive being split?"). Written here from the mathematics, in log space:

* each block i on its own gives ``lse_i = log sum_{allowed u in i} e^{s_u}`` (a
  logaddexp reduction, no running maximum) and its normalised output
  ``out_i = sum_u e^{s_u - lse_i} v_u``;
* over the union of blocks, ``lse = logaddexp(lse_1, ..., lse_k)`` and
  ``out = sum_i e^{lse_i - lse} out_i``, because each block's share of the union's
  normaliser is ``e^{lse_i - lse}``.

The partials are combined two at a time in the order given, so a test can check that
every order gives the full row. A block with no allowed key for a row has lse -inf and
contributes nothing; a row with no allowed key anywhere ends with output 0, lse -inf.
"""

from __future__ import annotations

import numpy as np


def block_partial(q, k, v, mask=None, scale=None):
    """One key block on its own: (out_i [R, dv], lse_i [R]) of the scaled scores
    ``q k^T * scale`` over the allowed keys (mask [R, n] bool, True = allowed)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if k.shape[0] == 0:
        return np.zeros((R, v.shape[1])), np.full(R, -np.inf)
    s = (q @ k.T) * scale
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    lse = np.logaddexp.reduce(s, axis=1)
    live = np.isfinite(lse)
    w = np.where(live[:, None], np.exp(s - np.where(live, lse, 0.0)[:, None]), 0.0)
    return w @ v, lse


def combine_partials(parts):
    """Results over disjoint key blocks [(out_i, lse_i), ...] combined, in list order,
    into the result over their union: lse = logaddexp of the lse_i, out = the sum of
    e^(lse_i - lse) out_i."""
    out, lse = None, None
    for o, l in parts:
        o = np.asarray(o, dtype=np.float64)
        l = np.asarray(l, dtype=np.float64)
        if out is None:
            out, lse = o.copy(), l.copy()
            continue
        tot = np.logaddexp(lse, l)
        live = np.isfinite(tot)
        ref = np.where(live, tot, 0.0)
        wa = np.where(live, np.exp(lse - ref), 0.0)
        wb = np.where(live, np.exp(l - ref), 0.0)
        out = wa[:, None] * out + wb[:, None] * o
        lse = tot
    out = np.where(np.isfinite(lse)[:, None], out, 0.0)
    return out, lse


def blockwise_attention(q, k_list, v_list, mask_list=None, scale=None):
    """Attention of q [R, d] over the blocks (k_list[i] [n_i, d], v_list[i] [n_i, dv],
    mask_list[i] [R, n_i] or None), built from each block's partial result and combined
    in list order. Returns (out [R, dv], lse [R])."""
    parts = []
    for i, (k, v) in enumerate(zip(k_list, v_list)):
        m = None if mask_list is None else mask_list[i]
        parts.append(block_partial(q, k, v, m, scale))
    return combine_partials(parts)
