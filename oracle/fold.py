"""Online-softmax fold over KV blocks, fp64: a second implementation used only to pin
the full-row oracle (``attention.rank_forward``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The update follows the rule described on "Ring Attention and Ulysses shard a sequence two
different ways, ...", section "Ring Attention: point-to-point rotation, and an online
softmax that never sees the whole row at once": keep, per query row, the largest score
seen so far, the sum of exponentials relative to it, and the un-normalised output; when a
block raises the maximum, rescale the sum and the output by e^(old max - new max) before
adding the block's own contribution; divide by the sum at the end. Written here over
masked blocks (a masked score is -inf) and with the 1/sqrt(d) scale applied to the
scores. A row with no allowed key in any block ends with output 0 and lse -inf.
"""

from __future__ import annotations

import numpy as np


def online_softmax_fold(q, k_list, v_list, mask_list=None, scale=None):
    """Fold the blocks (k_list[i], v_list[i]) into the running state in list order.

    q [R, d]; k_list[i] [n_i, d]; v_list[i] [n_i, dv]; mask_list[i] [R, n_i] bool
    (True = allowed) or None for all allowed. Returns (out [R, dv], lse [R]).
    """
    q = np.asarray(q, dtype=np.float64)
    R, d = q.shape
    dv = np.asarray(v_list[0]).shape[1] if len(v_list) else 0
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    best = np.full(R, -np.inf)       # largest allowed score so far
    norm = np.zeros(R)               # sum of exp(score - best) so far
    acc = np.zeros((R, dv))          # sum of exp(score - best) * v so far
    for i, (k, v) in enumerate(zip(k_list, v_list)):
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        s = (q @ k.T) * scale
        if mask_list is not None and mask_list[i] is not None:
            s = np.where(mask_list[i], s, -np.inf)
        blk_best = s.max(axis=1) if s.shape[1] else np.full(R, -np.inf)
        new_best = np.maximum(best, blk_best)
        live = np.isfinite(new_best)
        ref = np.where(live, new_best, 0.0)
        shrink = np.where(live, np.exp(best - ref), 1.0)   # e^(old - new); 0 when old = -inf
        w = np.exp(s - ref[:, None])                       # 0 for masked scores
        norm = norm * shrink + w.sum(axis=1)
        acc = acc * shrink[:, None] + w @ v
        best = new_best
    live = norm > 0
    out = np.where(live[:, None], acc / np.where(live, norm, 1.0)[:, None], 0.0)
    lse = np.where(live, best + np.log(np.where(live, norm, 1.0)), -np.inf)
    return out, lse
