"""Closed-form work and traffic counts for one rank's share (host logic, no GPU).

Counting convention: only allowed ("unmasked") score entries count, and each costs
4*d FLOP -- 2*d for its q.k dot product and 2*d for its share of P.V. Summed over the
full rows of every layer, forward and backward (3x the forward), this is the
"roughly 12 L h s FLOPs per token" of "What do you do about long sequences and sparse
models?", section "Why does the sequence need its own axis?".

Per-block allowed counts for rank i and KV block j (chunk size m = n/2 under zigzag,
n contiguous), derived from the zigzag pairing of "What breaks the load balance?":
  zigzag:      j != i -> 2 m^2;            j == i -> m^2 + m(m+1)
  contiguous:  j <  i -> n^2;  j == i -> n(n+1)/2;  j > i -> 0
  non-causal:  Nq * n
"""

from __future__ import annotations

import numpy as np


def block_allowed(c: int, rank: int, j: int, nq: int, n: int, causal: bool, zigzag: bool) -> int:
    """Allowed score entries of one (batch, query head) against KV block ``j``."""
    if not causal:
        return nq * n
    if zigzag:
        m = n // 2
        return m * m + m * (m + 1) if j == rank else 2 * m * m
    if j < rank:
        return n * n
    if j == rank:
        return n * (n + 1) // 2
    return 0


def allowed_entries(c: int, rank: int, nq: int, n: int, causal: bool, zigzag: bool,
                    round_begin: int = 0, round_end: int | None = None) -> int:
    """Allowed entries of one (batch, query head) over rounds [round_begin, round_end)."""
    if round_end is None:
        round_end = c
    return sum(block_allowed(c, rank, (rank - t) % c, nq, n, causal, zigzag)
               for t in range(round_begin, round_end))


def unmasked_flop(batch: int, hq: int, head_dim: int, entries_per_head: int) -> int:
    """FLOP counting only unmasked work: 4 * d per allowed entry, over all (b, h)."""
    return 4 * head_dim * entries_per_head * batch * hq


def needed_kv_rows(c: int, rank: int, j: int, n: int, causal: bool, zigzag: bool) -> int:
    """KV rows of block j that at least one of the rank's queries may attend to."""
    if not causal:
        return n
    if zigzag:
        m = n // 2
        # the early chunk j always precedes the rank's late chunk; the late chunk
        # 2c-1-j is reachable only when it does not follow the rank's late chunk
        return m + (m if j >= rank else 0)
    return n if j <= rank else 0


def algorithmic_bytes(batch: int, hq: int, hkv: int, nq: int, n: int, head_dim: int, elem_bytes: int,
                      c: int, rank: int, causal: bool, zigzag: bool, with_lse: bool = True,
                      round_begin: int = 0, round_end: int | None = None) -> int:
    """HBM bytes a launch must move at minimum: Q read once, each needed K/V row read
    once, the output written once, and the fp32 lse written once."""
    if round_end is None:
        round_end = c
    kv_rows = sum(needed_kv_rows(c, rank, (rank - t) % c, n, causal, zigzag)
                  for t in range(round_begin, round_end))
    q_bytes = batch * hq * nq * head_dim * elem_bytes
    kv_bytes = 2 * batch * hkv * kv_rows * head_dim * elem_bytes
    out_bytes = batch * hq * nq * head_dim * elem_bytes
    lse_bytes = 4 * batch * hq * nq if with_lse else 0
    return q_bytes + kv_bytes + out_bytes + lse_bytes


def merge_bytes(rows: int, head_dim: int, elem_bytes: int) -> int:
    """Minimum traffic of one merge: read two (out, lse) pairs, write one."""
    return 3 * rows * (head_dim * elem_bytes + 4)


def ring_break_even_tokens(flops_per_s: float, bytes_per_s: float) -> float:
    """Block size (tokens) at which one block's attention arithmetic (4 d c^2 FLOP)
    lasts as long as sending the next block (4 c d bytes): c >= F / B ("When is the
    ring actually free?"). The head dimension cancels."""
    return flops_per_s / bytes_per_s


def share_positions(c: int, rank: int, rows: int, zigzag: bool) -> np.ndarray:
    """Global positions of a rank's ``rows`` query rows: chunk ``rank`` of c, or (zigzag)
    chunks ``rank`` and 2c-1-rank of 2c, in row order."""
    if not zigzag:
        return rank * rows + np.arange(rows, dtype=np.int64)
    m = rows // 2
    return np.concatenate([rank * m + np.arange(m, dtype=np.int64),
                           (2 * c - 1 - rank) * m + np.arange(m, dtype=np.int64)])


def doc_allowed_entries(c: int, rank: int, rows: int, zigzag: bool, doc_start) -> int:
    """Allowed entries of one (batch, query head) over the whole ring under the document
    mask: the query at p sees the keys at doc_start[p] .. p, so it counts p - start + 1
    (none when the start lies past p)."""
    pos = share_positions(c, rank, rows, zigzag)
    lo = np.maximum(np.asarray(doc_start, dtype=np.int64)[pos], 0)
    return int(np.clip(pos - lo + 1, 0, None).sum())


def doc_needed_kv_rows(c: int, rank: int, rows: int, zigzag: bool, doc_start) -> int:
    """Key positions some query of the share may see under the document mask: the size
    of the union of the intervals [doc_start[p], p]."""
    S = c * rows
    pos = share_positions(c, rank, rows, zigzag)
    lo = np.maximum(np.asarray(doc_start, dtype=np.int64)[pos], 0)
    keep = lo <= pos
    cover = np.zeros(S + 1, dtype=np.int64)
    np.add.at(cover, lo[keep], 1)
    np.add.at(cover, pos[keep] + 1, -1)
    return int((np.cumsum(cover[:S]) > 0).sum())
