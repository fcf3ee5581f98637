"""Full-row fp64 oracle: what one rank's share of Ring Attention computes.

TEST INFRASTRUCTURE ONLY (see the package docstring). numpy, float64, CPU.

What is computed, and where it is stated:

* The ring is exact: folding the KV blocks in with a running max and running sum gives
  the same result as softmax over the whole row at once ("Ring Attention and Ulysses
  shard a sequence two different ways, ...", section "Ring Attention: point-to-point
  rotation, and an online softmax that never sees the whole row at once"; "What do you
  do about long sequences and sparse models?", section "How does attention survive
  being split?"). So the oracle is the plain definition, over the full row:
  ``softmax(q k^T / sqrt(d) + mask) v``, with no online update and no blocking beyond
  bounding memory by query rows.
* The scale ``1/sqrt(d)`` (d = head dimension) is the standard attention scale; the
  page's numpy sketch leaves it out (it multiplies raw ``q @ k.T``), and the tiny
  worked example (q 4x8, k/v 12x8) is reproduced here with the scale included.
* Causal mask: token i attends to every token j <= i ("Context & Expert Parallelism",
  section "Context parallelism: splitting the sequence").
* Zigzag ownership: cut the sequence into 2c chunks and give rank i chunks i and
  2c-1-i ("What do you do about long sequences and sparse models?", section "What
  breaks the load balance?"). Reading taken: a rank's rows are chunk i followed by
  chunk 2c-1-i; KV block j (rank j's keys/values) is laid out the same way.
* Ring order: round 0 is the local block, round r the block from r hops back ("Ring
  Attention: point-to-point rotation, ..."): block ``(rank - r) mod c``. The value does
  not depend on the order; only the set of blocks in a round range matters.
* GQA: fewer KV heads than query heads ("What do you do about long sequences and sparse
  models?", section "Why did Llama 3 not use a ring?"). Reading taken: query head h uses
  KV head ``h // (Hq / Hkv)``.
* Log-sum-exp per row: ``lse = ln sum_allowed exp(s)`` of the scaled scores, natural
  log; ``-inf`` (with output 0) for a row with no allowed key.
* Document mask: in a packed sequence, attention must not cross document boundaries
  ("What do you do about long sequences and sparse models?", section "Why did Llama 3
  not use a ring?"). Reading taken: documents are contiguous spans; ``doc_start[p]`` is
  the global position where p's document begins (so it also identifies the document),
  and the query at p sees exactly the keys at positions x with doc_start[p] <= x <= p.
  Values of ``doc_start`` are taken as given (a value above p leaves the row empty).
"""

from __future__ import annotations

import numpy as np

# Rows of scores materialised at once, to bound memory (rows x keys x 8 bytes).
_SCORE_BUDGET = 1 << 25


def score_scale(d: int) -> float:
    """Scale applied to q.k before the softmax: 1/sqrt(d), d = head dimension."""
    return 1.0 / np.sqrt(d)


def causal_allowed(pos_q: np.ndarray, pos_k: np.ndarray) -> np.ndarray:
    """[len(pos_q), len(pos_k)] mask of the causal rule: key j is visible to query i iff
    j <= i ("Context parallelism: splitting the sequence")."""
    return pos_k[None, :] <= pos_q[:, None]


def document_allowed(pos_q: np.ndarray, pos_k: np.ndarray, doc_start) -> np.ndarray:
    """[len(pos_q), len(pos_k)] mask of the causal document rule: the query at p sees the
    key at x iff doc_start[p] <= x <= p (its own document, up to itself)."""
    lo = np.asarray(doc_start, dtype=np.int64)[pos_q]
    return (pos_k[None, :] <= pos_q[:, None]) & (pos_k[None, :] >= lo[:, None])


def kv_head(h: int, hq: int, hkv: int) -> int:
    """KV head used by query head ``h`` (grouped-query attention)."""
    return h // (hq // hkv)


def chunk_positions(owner: int, rows: int, c: int, zigzag: bool) -> np.ndarray:
    """Global token positions of the ``rows`` rows held by ``owner`` (a rank's queries,
    or KV block ``owner``).

    Contiguous: the sequence is cut into c chunks of ``rows`` tokens and owner i holds
    chunk i. Zigzag: the sequence is cut into 2c chunks of ``rows/2`` tokens and owner i
    holds chunk i then chunk 2c-1-i ("What breaks the load balance?").
    """
    t = np.arange(rows, dtype=np.int64)
    if not zigzag:
        return owner * rows + t
    if rows % 2:
        raise ValueError("zigzag needs an even number of rows per owner")
    m = rows // 2
    first = owner * m + t[:m]
    second = (2 * c - 1 - owner) * m + t[:m]
    return np.concatenate([first, second])


def ring_blocks(c: int, rank: int, round_begin: int = 0, round_end: int | None = None):
    """KV blocks a rank folds in during rounds [round_begin, round_end): round r uses the
    block that has travelled r hops, i.e. block (rank - r) mod c."""
    if round_end is None:
        round_end = c
    return [(rank - r) % c for r in range(round_begin, round_end)]


def _row_attention(qrows, kall, vall, allowed, scale):
    """Softmax attention of each query row over the allowed keys, in fp64.

    qrows [R, d]; kall [S, d]; vall [S, dv]; allowed [R, S] bool.
    Returns out [R, dv], lse [R].
    """
    s = (qrows @ kall.T) * scale
    s = np.where(allowed, s, -np.inf)
    mx = s.max(axis=1)
    any_allowed = np.isfinite(mx)
    mx_safe = np.where(any_allowed, mx, 0.0)
    w = np.exp(s - mx_safe[:, None])  # masked entries give exp(-inf) = 0
    tot = w.sum(axis=1)
    lse = np.where(any_allowed, mx_safe + np.log(np.where(any_allowed, tot, 1.0)), -np.inf)
    out = (w @ vall) / np.where(any_allowed, tot, 1.0)[:, None]
    out[~any_allowed] = 0.0
    return out, lse


def rank_forward(q, k_blocks, v_blocks, c: int, rank: int, causal: bool, zigzag: bool,
                 round_begin: int = 0, round_end: int | None = None, rows=None, doc_start=None):
    """Oracle for one rank's share: attention of the rank's queries over the keys of the
    KV blocks it folds in during rounds [round_begin, round_end) (all c rounds by
    default, which is the full row).

    q        [B, Hq, Nq, d]      the rank's queries (any float dtype; upcast to fp64)
    k_blocks [c, B, Hkv, n, d]   KV block j = rank j's keys, in owner order
    v_blocks [c, B, Hkv, n, dv]
    rows     optional int array [R, 3] of (b, h, t) triples: compute only those rows.
    doc_start optional int array [c * n] by global position (causal only): the document
             mask, keys at doc_start[p] <= x <= p for the query at p.

    Returns (out, lse): out [B, Hq, Nq, dv] fp64 and lse [B, Hq, Nq] fp64 when rows is
    None, else out [R, dv] and lse [R] in the order of ``rows``.
    """
    q = np.asarray(q, dtype=np.float64)
    k_blocks = np.asarray(k_blocks, dtype=np.float64)
    v_blocks = np.asarray(v_blocks, dtype=np.float64)
    B, hq, nq, d = q.shape
    cc, b2, hkv, n, d2 = k_blocks.shape
    if cc != c or b2 != B or d2 != d or v_blocks.shape[:4] != k_blocks.shape[:4]:
        raise ValueError("shape mismatch")
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and nq != n:
        raise ValueError("causal needs as many query rows as KV rows per block")
    if doc_start is not None:
        if not causal:
            raise ValueError("the document mask is causal")
        doc_start = np.asarray(doc_start, dtype=np.int64)
        if doc_start.shape != (c * n,):
            raise ValueError("doc_start needs one entry per global position (c * n)")
    dv = v_blocks.shape[4]
    scale = score_scale(d)

    blocks = ring_blocks(c, rank, round_begin, round_end)
    pos_q = chunk_positions(rank, nq, c, zigzag) if causal else None
    if blocks:
        pos_k = np.concatenate([chunk_positions(j, n, c, zigzag) for j in blocks]) if causal else None
    else:
        pos_k = np.zeros(0, dtype=np.int64)

    def kv_for(b, g):
        if not blocks:
            return np.zeros((0, d)), np.zeros((0, dv))
        return (np.concatenate([k_blocks[j, b, g] for j in blocks]),
                np.concatenate([v_blocks[j, b, g] for j in blocks]))

    def attend(b, h, ts):
        kall, vall = kv_for(b, kv_head(h, hq, hkv))
        if kall.shape[0] == 0:
            return np.zeros((len(ts), dv)), np.full(len(ts), -np.inf)
        outs, lses = [], []
        step = max(1, _SCORE_BUDGET // max(1, kall.shape[0]))
        for i in range(0, len(ts), step):
            tt = ts[i:i + step]
            if doc_start is not None:
                allowed = document_allowed(pos_q[tt], pos_k, doc_start)
            elif causal:
                allowed = causal_allowed(pos_q[tt], pos_k)
            else:
                allowed = np.ones((len(tt), kall.shape[0]), dtype=bool)
            o, l = _row_attention(q[b, h, tt], kall, vall, allowed, scale)
            outs.append(o)
            lses.append(l)
        return np.concatenate(outs), np.concatenate(lses)

    if rows is None:
        out = np.zeros((B, hq, nq, dv))
        lse = np.zeros((B, hq, nq))
        ts = np.arange(nq)
        for b in range(B):
            for h in range(hq):
                if nq:
                    out[b, h], lse[b, h] = attend(b, h, ts)
        return out, lse

    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.zeros((len(rows), dv))
    lse = np.zeros(len(rows))
    for b in range(B):
        for h in range(hq):
            sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
            if len(sel):
                out[sel], lse[sel] = attend(b, h, rows[sel, 2])
    return out, lse


def merge(out_a, lse_a, out_b, lse_b):
    """Combine two partial results of attention over disjoint key sets into the result
    over their union ("How does attention survive being split?": partial results over
    different key blocks combine exactly through their running max and sum).

    Each partial is (normalised output, lse). With M = max(lse_a, lse_b), the weights
    e^(lse_a - M) and e^(lse_b - M) are each side's share of the union's normaliser.
    A side with lse = -inf holds no keys and contributes nothing; both -inf gives
    (0, -inf). Shapes: out [..., dv], lse [...].
    """
    out_a = np.asarray(out_a, dtype=np.float64)
    out_b = np.asarray(out_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    wa = np.exp(la - m_safe)
    wb = np.exp(lb - m_safe)
    tot = wa + wb
    tot_safe = np.where(empty, 1.0, tot)
    out = (wa[..., None] * out_a + wb[..., None] * out_b) / tot_safe[..., None]
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))
    return out, lse


def allowed_count(c: int, rank: int, rows: int, causal: bool, zigzag: bool,
                  round_begin: int = 0, round_end: int | None = None, doc_start=None) -> int:
    """Brute-force count of allowed (query, key) score entries for one (batch, head) of
    rank ``rank``'s share, where each owner holds ``rows`` rows (Nq = n = rows)."""
    blocks = ring_blocks(c, rank, round_begin, round_end)
    if not causal:
        return rows * rows * len(blocks)
    pq = chunk_positions(rank, rows, c, zigzag)
    total = 0
    for j in blocks:
        pk = chunk_positions(j, rows, c, zigzag)
        m = causal_allowed(pq, pk) if doc_start is None else document_allowed(pq, pk, doc_start)
        total += int(m.sum())
    return total


def chunk_units(c: int, rank: int, zigzag: bool) -> int:
    """Units of causal work of one rank, as the load-balance argument counts them: the
    number of (query chunk, key chunk) pairs in which at least one score entry is
    allowed ("What breaks the load balance?")."""
    chunks = 2 * c if zigzag else c
    size = 2  # two tokens per chunk is enough to see the chunk pattern
    rows = size * (2 if zigzag else 1)
    pq = chunk_positions(rank, rows, c, zigzag)
    q_chunks = sorted({int(p) // size for p in pq})
    units = 0
    for qc in q_chunks:
        qpos = np.arange(qc * size, (qc + 1) * size)
        for kc in range(chunks):
            kpos = np.arange(kc * size, (kc + 1) * size)
            if causal_allowed(qpos, kpos).any():
                units += 1
    return units
