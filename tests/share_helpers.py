"""Test-side construction of rank shares from a global sequence.

Written independently of the oracle's position arithmetic: ownership is expressed by
cutting ``arange(S)`` with ``numpy.array_split`` into c (contiguous) or 2c (zigzag)
chunks and handing rank i chunk i, or chunks i and 2c-1-i ("What do you do about long
sequences and sparse models?", section "What breaks the load balance?").
"""

from __future__ import annotations

import numpy as np


def owned_positions(S: int, c: int, zigzag: bool):
    """List over owners of the global positions each holds, in row order."""
    if zigzag:
        chunks = np.array_split(np.arange(S), 2 * c)
        return [np.concatenate([chunks[i], chunks[2 * c - 1 - i]]) for i in range(c)]
    return np.array_split(np.arange(S), c)


def build_share(qg, kg, vg, c: int, rank: int, zigzag: bool):
    """From global q [B,Hq,S,d], k/v [B,Hkv,S,d] build the rank's q [B,Hq,Nq,d] and the
    stacked KV blocks [c,B,Hkv,n,d] in owner order. Returns (q, k_blocks, v_blocks, own)."""
    own = owned_positions(qg.shape[2], c, zigzag)
    q = qg[:, :, own[rank]]
    kb = np.stack([kg[:, :, own[j]] for j in range(c)])
    vb = np.stack([vg[:, :, own[j]] for j in range(c)])
    return q, kb, vb, own


def expand_gqa(kg, hq: int):
    """Repeat each KV head hq/hkv times along the head axis (query head h reads KV head
    h // (hq/hkv)), the convention of torch's enable_gqa."""
    return np.repeat(kg, hq // kg.shape[1], axis=1)
