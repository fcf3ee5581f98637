"""Pins of the fp64 oracle to things other than itself (CPU only).

* 50-digit brute force on tiny inputs, every mode (mask, zigzag, GQA).
* Attention rebuilt from per-block partial results (each block's own softmax, combined
  with logaddexp weights) in every block order, and on unequal re-splits.
* The pages' worked example (q 4x8, k/v 12x8, 3 blocks; allclose at atol 1e-6).
* torch's fp64 scaled_dot_product_attention (is_causal, enable_gqa) on the full sequence.
* Zigzag/contiguous shares gathered out of full-sequence causal attention.
* Closed forms: Q = 0, constant V, a common shift of every key.
* Merge algebra and per-round partials merged back into the fused result.
* Ring direction: rank i sends its block to rank i+1.
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from tests.share_helpers import build_share, expand_gqa, owned_positions

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _global(B, hq, hkv, S, d, seed, scale=1.0):
    r = _rng(seed)
    return (r.standard_normal((B, hq, S, d)) * scale,
            r.standard_normal((B, hkv, S, d)) * scale,
            r.standard_normal((B, hkv, S, d)) * scale)


# --------------------------------------------------------------------------- T1
def _mp_bruteforce(qg, kg, vg, causal):
    """Direct sum_u e^{s_u} v_u / sum_u e^{s_u} at 50 digits, no max subtraction, over
    every global key position u (<= the query position when causal)."""
    import mpmath as mp
    mp.mp.dps = 50
    B, hq, S, d = qg.shape
    kx, vx = expand_gqa(kg, hq), expand_gqa(vg, hq)
    inv = 1 / mp.sqrt(d)
    out = np.zeros(qg.shape)
    lse = np.zeros(qg.shape[:3])
    for b in range(B):
        for h in range(hq):
            for p in range(S):
                keys = range(p + 1) if causal else range(S)
                w = [mp.exp(mp.fsum(mp.mpf(float(qg[b, h, p, i])) * mp.mpf(float(kx[b, h, u, i]))
                                    for i in range(d)) * inv) for u in keys]
                z = mp.fsum(w)
                lse[b, h, p] = float(mp.log(z))
                for e in range(d):
                    out[b, h, p, e] = float(mp.fsum(wu * mp.mpf(float(vx[b, h, u, e]))
                                                    for wu, u in zip(w, keys)) / z)
    return out, lse


@pytest.mark.parametrize("causal,zigzag,hq,hkv,c,S", [
    (False, False, 1, 1, 3, 12),
    (True, False, 2, 1, 4, 16),
    (True, True, 2, 2, 2, 16),
    (True, True, 4, 2, 4, 16),
])
def test_t1_bruteforce_50_digits(causal, zigzag, hq, hkv, c, S):
    d = 4
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=11 + c + hq)
    ref_out, ref_lse = _mp_bruteforce(qg, kg, vg, causal)
    for rank in range(c):
        q, kb, vb, own = build_share(qg, kg, vg, c, rank, zigzag)
        out, lse = oracle.rank_forward(q, kb, vb, c, rank, causal, zigzag)
        np.testing.assert_allclose(out, ref_out[:, :, own[rank]], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse[:, :, own[rank]], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- T2
def test_page_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "ring_example.json")))
    r = _rng(0)
    q = r.standard_normal(g["q_shape"])
    kf = r.standard_normal(g["kv_shape"])
    vf = r.standard_normal(g["kv_shape"])
    nb = g["blocks"]
    kb = np.stack(np.split(kf, nb))[:, None, None]
    vb = np.stack(np.split(vf, nb))[:, None, None]
    full, _ = oracle.rank_forward(q[None, None], kb, vb, nb, 0, False, False)
    ring, _ = oracle.blockwise_attention(q, np.split(kf, nb), np.split(vf, nb))
    assert np.allclose(full[0, 0], ring, atol=g["atol"]) == g["expected_allclose"]
    np.testing.assert_allclose(full[0, 0], ring, rtol=0, atol=1e-13)


def _share_blocks_with_masks(qg, kg, vg, c, rank, zigzag, causal, b, h):
    """Per-block (k, v, mask) lists for one (b, h) of a rank, masks from global positions."""
    own = owned_positions(qg.shape[2], c, zigzag)
    g = h // (qg.shape[1] // kg.shape[1])
    pq = own[rank]
    ks, vs, ms = [], [], []
    for j in range(c):
        ks.append(kg[b, g, own[j]])
        vs.append(vg[b, g, own[j]])
        ms.append(own[j][None, :] <= pq[:, None] if causal else None)
    return qg[b, h, pq], ks, vs, ms


@pytest.mark.parametrize("causal,zigzag", [(False, False), (True, False), (True, True)])
def test_t2_blockwise_any_order_equals_full_row(causal, zigzag):
    c, S, d, hq, hkv = 4, 32, 8, 2, 1
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=5)
    for rank in range(c):
        q, kb, vb, own = build_share(qg, kg, vg, c, rank, zigzag)
        full_out, full_lse = oracle.rank_forward(q, kb, vb, c, rank, causal, zigzag)
        for h in range(hq):
            qr, ks, vs, ms = _share_blocks_with_masks(qg, kg, vg, c, rank, zigzag, causal, 0, h)
            for order in itertools.permutations(range(c)):
                o, l = oracle.blockwise_attention(qr, [ks[i] for i in order], [vs[i] for i in order],
                                                  [ms[i] for i in order])
                np.testing.assert_allclose(o, full_out[0, h], rtol=0, atol=1e-12)
                np.testing.assert_allclose(l, full_lse[0, h], rtol=0, atol=1e-12)


def test_t2_blockwise_unequal_resplits():
    c, S, d = 6, 48, 8
    qg, kg, vg = _global(1, 1, 1, S, d, seed=7)
    r = _rng(70)
    for rank in range(c):
        q, kb, vb, own = build_share(qg, kg, vg, c, rank, True)
        full_out, full_lse = oracle.rank_forward(q, kb, vb, c, rank, True, True)
        allk = kg[0, 0]
        allv = vg[0, 0]
        mask = np.arange(S)[None, :] <= own[rank][:, None]
        for _ in range(20):
            perm = r.permutation(S)
            cuts = np.sort(r.choice(np.arange(1, S), size=r.integers(1, 8), replace=False))
            parts = np.split(perm, cuts)
            o, l = oracle.blockwise_attention(q[0, 0], [allk[p] for p in parts], [allv[p] for p in parts],
                                              [mask[:, p] for p in parts])
            np.testing.assert_allclose(o, full_out[0, 0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(l, full_lse[0, 0], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- T4/T5
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (8, 1)])
def test_t5_torch_sdpa_fp64(hq, hkv):
    import torch
    import torch.nn.functional as F
    S, d = 64, 16
    qg, kg, vg = _global(2, hq, hkv, S, d, seed=hq * 10 + hkv)
    for causal in (False, True):
        ref = F.scaled_dot_product_attention(torch.from_numpy(qg), torch.from_numpy(kg), torch.from_numpy(vg),
                                             is_causal=causal, enable_gqa=True).numpy()
        # c = 1: the full sequence is the rank's share
        out, _ = oracle.rank_forward(qg, kg[None], vg[None], 1, 0, causal, False)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("zigzag", [False, True])
def test_t4_share_rows_equal_full_sequence_rows(zigzag):
    import torch
    import torch.nn.functional as F
    c, S, d, hq, hkv = 4, 64, 8, 4, 2
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=3)
    ref = F.scaled_dot_product_attention(torch.from_numpy(qg), torch.from_numpy(kg), torch.from_numpy(vg),
                                         is_causal=True, enable_gqa=True).numpy()
    for rank in range(c):
        q, kb, vb, own = build_share(qg, kg, vg, c, rank, zigzag)
        out, _ = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag)
        np.testing.assert_allclose(out, ref[:, :, own[rank]], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------- T6
@pytest.mark.parametrize("zigzag", [False, True])
def test_t6_closed_forms(zigzag):
    c, S, d, hq, hkv = 4, 128, 16, 4, 2
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=9)
    for rank in range(c):
        own = owned_positions(S, c, zigzag)[rank]
        # Q = 0: uniform weights over the allowed keys
        q, kb, vb, _ = build_share(np.zeros_like(qg), kg, vg, c, rank, zigzag)
        out, lse = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag)
        np.testing.assert_allclose(lse[0], np.broadcast_to(np.log(own + 1.0), lse[0].shape), rtol=0, atol=1e-13)
        prefix_mean = np.cumsum(expand_gqa(vg, hq), axis=2) / (np.arange(S) + 1.0)[None, None, :, None]
        np.testing.assert_allclose(out, prefix_mean[:, :, own], rtol=0, atol=1e-13)
        # constant V per KV head: the output is that constant
        vc = np.broadcast_to(np.arange(hkv, dtype=np.float64)[None, :, None, None] + 0.5, vg.shape)
        q, kb, vb, _ = build_share(qg, kg, vc, c, rank, zigzag)
        out, _ = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag)
        expect = (np.arange(hq) // (hq // hkv) + 0.5)[None, :, None, None]
        np.testing.assert_allclose(out, np.broadcast_to(expect, out.shape), rtol=0, atol=1e-13)
        # a common shift u of every key: output unchanged, lse moves by q.u / sqrt(d)
        u = _rng(rank).standard_normal(d)
        q, kb, vb, _ = build_share(qg, kg, vg, c, rank, zigzag)
        o1, l1 = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag)
        o2, l2 = oracle.rank_forward(q, kb + u, vb, c, rank, True, zigzag)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l1 + (q @ u) / np.sqrt(d), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- T7
def test_t7_merge_algebra():
    r = _rng(1)
    oa, ob = r.standard_normal((50, 8)), r.standard_normal((50, 8))
    la, lb = r.standard_normal(50) * 5, r.standard_normal(50) * 5
    la[3] = -np.inf
    lb[4] = -np.inf
    la[5] = lb[5] = -np.inf
    m1 = oracle.merge(oa, la, ob, lb)
    m2 = oracle.merge(ob, lb, oa, la)
    assert np.array_equal(m1[0], m2[0]) and np.array_equal(m1[1], m2[1])
    ident = oracle.merge(oa, la, np.zeros_like(oa), np.full(50, -np.inf))
    fin = np.isfinite(la)
    assert np.array_equal(ident[0][fin], oa[fin]) and np.array_equal(ident[1], la)
    assert np.all(m1[0][5] == 0) and m1[1][5] == -np.inf
    np.testing.assert_allclose(m1[0][3], ob[3], rtol=0, atol=0)


@pytest.mark.parametrize("causal,zigzag", [(False, False), (True, False), (True, True)])
def test_t7_partials_merge_to_fused(causal, zigzag):
    c, S, d, hq, hkv = 4, 64, 8, 4, 2
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=21)
    for rank in range(c):
        q, kb, vb, _ = build_share(qg, kg, vg, c, rank, zigzag)
        fused = oracle.rank_forward(q, kb, vb, c, rank, causal, zigzag)
        acc = oracle.rank_forward(q, kb, vb, c, rank, causal, zigzag, 0, 1)
        for t in range(1, c):
            part = oracle.rank_forward(q, kb, vb, c, rank, causal, zigzag, t, t + 1)
            acc = oracle.merge(*acc, *part)
        np.testing.assert_allclose(acc[0], fused[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(acc[1], fused[1], rtol=0, atol=1e-12)
        split = oracle.merge(*oracle.rank_forward(q, kb, vb, c, rank, causal, zigzag, 0, 2),
                             *oracle.rank_forward(q, kb, vb, c, rank, causal, zigzag, 2, c))
        np.testing.assert_allclose(split[0], fused[0], rtol=0, atol=1e-12)


def test_partial_round_fully_masked_rows():
    # rank 0, zigzag: its early chunk sees nothing in any block but its own
    c, S, d = 4, 32, 4
    qg, kg, vg = _global(1, 1, 1, S, d, seed=2)
    q, kb, vb, own = build_share(qg, kg, vg, c, 0, True)
    out, lse = oracle.rank_forward(q, kb, vb, c, 0, True, True, 1, 2)
    m = S // (2 * c)
    assert np.all(lse[0, 0, :m] == -np.inf) and np.all(out[0, 0, :m] == 0)
    assert np.all(np.isfinite(lse[0, 0, m:]))


# --------------------------------------------------------------------------- ring order
def test_ring_direction_rank_i_sends_to_i_plus_1():
    for c in (1, 2, 5, 8):
        for i in range(c):
            assert A.ring_blocks(c, i, 0, 1) == [i]            # round 0 is local
            for t in range(1, c):
                # the block rank i holds in round t is what rank i-1 held in round t-1
                assert A.ring_blocks(c, i, t, t + 1) == A.ring_blocks(c, (i - 1) % c, t - 1, t)
            assert sorted(A.ring_blocks(c, i)) == list(range(c))


def test_sampled_rows_match_full():
    c, S, d, hq, hkv = 4, 64, 8, 4, 2
    qg, kg, vg = _global(2, hq, hkv, S, d, seed=8)
    q, kb, vb, _ = build_share(qg, kg, vg, c, 1, True)
    out, lse = oracle.rank_forward(q, kb, vb, c, 1, True, True)
    rows = np.array([[0, 0, 0], [1, 3, 15], [0, 2, 7], [1, 1, 8]])
    o, l = oracle.rank_forward(q, kb, vb, c, 1, True, True, rows=rows)
    # same arithmetic on a different row grouping: equal up to BLAS rounding
    np.testing.assert_allclose(o, out[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, lse[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- T8
# Document mask of packed sequences ("Why did Llama 3 not use a ring?"): the query at p
# sees the keys of its own document up to itself.
def _docs(S, lengths):
    from blockwise_ring_attention_amd.inputs import doc_start_from_lengths
    assert sum(lengths) == S
    return doc_start_from_lengths(lengths)


DOC_LAYOUTS = [[64], [1, 63], [10, 1, 1, 20, 32], [17, 15, 16, 16], [5] * 12 + [4]]


@pytest.mark.parametrize("lengths", DOC_LAYOUTS)
def test_t8_documents_equal_separate_causal_attention(lengths):
    """Each document attends like an independent causal sequence: torch's fp64 causal
    attention on every document span separately equals the oracle's rows (c = 1)."""
    import torch
    import torch.nn.functional as F
    S, d, hq, hkv = 64, 8, 4, 2
    qg, kg, vg = _global(2, hq, hkv, S, d, seed=81)
    ds = _docs(S, lengths)
    out, lse = oracle.rank_forward(qg, kg[None], vg[None], 1, 0, True, False, doc_start=ds)
    a = 0
    for n in lengths:
        sl = slice(a, a + n)
        ref = F.scaled_dot_product_attention(torch.from_numpy(qg[:, :, sl]), torch.from_numpy(kg[:, :, sl]),
                                             torch.from_numpy(vg[:, :, sl]), is_causal=True, enable_gqa=True).numpy()
        np.testing.assert_allclose(out[:, :, sl], ref, rtol=0, atol=1e-13)
        a += n


def _mp_doc_bruteforce(qg, kg, vg, ds):
    import mpmath as mp
    mp.mp.dps = 50
    B, hq, S, d = qg.shape
    kx, vx = expand_gqa(kg, hq), expand_gqa(vg, hq)
    inv = 1 / mp.sqrt(d)
    out = np.zeros(qg.shape)
    lse = np.zeros(qg.shape[:3])
    for b in range(B):
        for h in range(hq):
            for p in range(S):
                keys = range(int(ds[p]), p + 1)
                w = [mp.exp(mp.fsum(mp.mpf(float(qg[b, h, p, i])) * mp.mpf(float(kx[b, h, u, i]))
                                    for i in range(d)) * inv) for u in keys]
                z = mp.fsum(w)
                lse[b, h, p] = float(mp.log(z))
                for e in range(d):
                    out[b, h, p, e] = float(mp.fsum(wu * mp.mpf(float(vx[b, h, u, e]))
                                                    for wu, u in zip(w, keys)) / z)
    return out, lse


@pytest.mark.parametrize("zigzag", [False, True])
def test_t8_documents_bruteforce_50_digits(zigzag):
    S, d, hq, hkv, c = 16, 4, 2, 1, 2
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=83)
    ds = _docs(S, [3, 1, 7, 5])
    ref_out, ref_lse = _mp_doc_bruteforce(qg, kg, vg, ds)
    for rank in range(c):
        q, kb, vb, own = build_share(qg, kg, vg, c, rank, zigzag)
        out, lse = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag, doc_start=ds)
        np.testing.assert_allclose(out, ref_out[:, :, own[rank]], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse[:, :, own[rank]], rtol=0, atol=1e-13)


@pytest.mark.parametrize("zigzag", [False, True])
def test_t8_one_document_is_the_causal_mask(zigzag):
    c, S, d, hq, hkv = 4, 64, 8, 4, 2
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=85)
    for rank in range(c):
        q, kb, vb, _ = build_share(qg, kg, vg, c, rank, zigzag)
        a = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag)
        b = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag, doc_start=np.zeros(S, dtype=np.int32))
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("zigzag", [False, True])
def test_t8_document_shares_and_closed_form(zigzag):
    """Shares gathered out of the full sequence, and Q = 0: uniform weights over the
    document prefix, so lse = ln(p - start + 1) and out = the mean of those V rows."""
    c, S, d, hq, hkv = 4, 64, 8, 4, 2
    qg, kg, vg = _global(1, hq, hkv, S, d, seed=87)
    ds = _docs(S, [9, 23, 1, 2, 29])
    full, _ = oracle.rank_forward(qg, kg[None], vg[None], 1, 0, True, False, doc_start=ds)
    vx = expand_gqa(vg, hq)
    for rank in range(c):
        q, kb, vb, own = build_share(qg, kg, vg, c, rank, zigzag)
        out, _ = oracle.rank_forward(q, kb, vb, c, rank, True, zigzag, doc_start=ds)
        np.testing.assert_allclose(out, full[:, :, own[rank]], rtol=0, atol=1e-13)
        q0, _, _, _ = build_share(np.zeros_like(qg), kg, vg, c, rank, zigzag)
        out0, lse0 = oracle.rank_forward(q0, kb, vb, c, rank, True, zigzag, doc_start=ds)
        pos = own[rank]
        np.testing.assert_allclose(lse0[0], np.broadcast_to(np.log(pos - ds[pos] + 1.0), lse0[0].shape),
                                   rtol=0, atol=1e-13)
        for i, p in enumerate(pos):
            np.testing.assert_allclose(out0[0, :, i], vx[0, :, ds[p]:p + 1].mean(axis=1), rtol=0, atol=1e-13)


def test_t8_document_allowed_counts():
    """The brute-force allowed count with documents is sum over rows of p - start + 1."""
    c, rows = 4, 16
    S = c * rows
    ds = _docs(S, [9, 23, 1, 2, 29])
    for zigzag in (False, True):
        total = sum(oracle.allowed_count(c, r, rows, True, zigzag, doc_start=ds) for r in range(c))
        assert total == int(np.sum(np.arange(S) - ds + 1))


def test_t7_merge_equals_logspace_combination():
    """oracle.merge against the log-space combination of two partials (written apart from
    it in oracle/fold.py), on random partials with empty rows on either or both sides."""
    r = _rng(77)
    R, dv = 64, 8
    oa, ob = r.standard_normal((R, dv)), r.standard_normal((R, dv))
    la, lb = r.standard_normal(R) * 5, r.standard_normal(R) * 5
    la[:8] = -np.inf
    lb[4:12] = -np.inf
    oa[:8] = 0.0
    ob[4:12] = 0.0
    got_o, got_l = oracle.merge(oa, la, ob, lb)
    ref_o, ref_l = oracle.combine_partials([(oa, la), (ob, lb)])
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_o, ref_o, rtol=0, atol=1e-13)
    assert np.all(got_o[4:8] == 0.0) and np.all(np.isneginf(got_l[4:8]))   # empty on both sides
