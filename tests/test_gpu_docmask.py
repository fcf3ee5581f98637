"""GPU parity of the document mask of packed sequences (ra_rank_forward_doc, through the
C ABI) against the fp64 oracle: the query at global position p sees the keys at
doc_start[p] <= x <= p ("What do you do about long sequences and sparse models?",
section "Why did Llama 3 not use a ring?").

Small cases compare every element: packed documents of mixed lengths (1-token documents,
documents crossing chunk and tile edges), a single document (the causal mask), every
token its own document, start values that are not monotone, and start values past the
query (rows without keys); both dtypes, zigzag and contiguous ownership, round ranges.
The 128k packed-document workload is checked on sampled rows and, over every row, by
the Q = 0 closed form (uniform weights over the document prefix); its streamed form (one
accumulating launch per round) on sampled rows and, over every row, against the fused
launch's lse."""

import numpy as np
import pytest

import oracle
from blockwise_ring_attention_amd.inputs import (WORKLOADS, doc_start_from_lengths, draw_document_lengths,
                                                  make_doc_start, make_inputs, random_array)
from tests.gpu_util import assert_parity, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


def run_gpu_doc(q, k, v, ds, c, rank, zigzag, t0=0, t1=None, dtype="bf16", with_lse=True):
    import torch
    import blockwise_ring_attention_amd as ra
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    dd = torch.from_numpy(np.ascontiguousarray(ds, dtype=np.int32)).cuda()
    out, lse = ra.rank_forward_doc(qd, kd, vd, dd, c, rank, zigzag, t0, t1, with_lse=with_lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64) if lse is not None else None
    return o, l


def _layout(kind, S, seed):
    rng = np.random.default_rng(seed)
    if kind == "packed":
        return doc_start_from_lengths(draw_document_lengths(S, 37, 1.2, seed))
    if kind == "single":
        return np.zeros(S, dtype=np.int32)
    if kind == "tokens":
        return np.arange(S, dtype=np.int32)
    if kind == "nonmono":
        return (rng.integers(0, np.arange(S) + 1)).astype(np.int32)
    if kind == "beyond":
        ds = doc_start_from_lengths(draw_document_lengths(S, 50, 1.0, seed)).astype(np.int64)
        pick = rng.random(S) < 0.05
        ds[pick] = np.arange(S)[pick] + 1 + rng.integers(0, 5, pick.sum())
        return ds.astype(np.int32)
    if kind == "extreme":
        # starts at or before the sequence start (negative, down to INT32_MIN) see every key
        # up to the query; starts past the sequence end (up to INT32_MAX) see none
        ds = doc_start_from_lengths(draw_document_lengths(S, 40, 1.0, seed)).astype(np.int64)
        u = rng.random(S)
        ds[u < 0.10] = np.iinfo(np.int32).min
        ds[(u >= 0.10) & (u < 0.20)] = -rng.integers(1, 1000, ((u >= 0.10) & (u < 0.20)).sum())
        ds[(u >= 0.20) & (u < 0.25)] = np.iinfo(np.int32).max
        ds[(u >= 0.25) & (u < 0.30)] = S + rng.integers(0, 1000, ((u >= 0.25) & (u < 0.30)).sum())
        return ds.astype(np.int32)
    raise ValueError(kind)


CASES = [
    # B, hq, hkv, d, n, c, rank, zigzag, dtype, layout
    (1, 8, 1, 128, 512, 4, 0, True, "bf16", "packed"),
    (1, 8, 2, 128, 512, 4, 3, True, "bf16", "packed"),
    (1, 4, 1, 128, 200, 3, 1, True, "bf16", "packed"),     # ragged chunks (m = 100)
    (2, 6, 2, 64, 136, 4, 2, False, "bf16", "packed"),     # contiguous, G = 3, d = 64
    (1, 16, 1, 128, 96, 2, 1, True, "bf16", "packed"),     # two head sets
    (1, 4, 2, 128, 256, 4, 1, True, "bf16", "single"),
    (1, 4, 2, 128, 256, 4, 2, True, "bf16", "tokens"),
    (1, 8, 1, 128, 384, 3, 2, True, "bf16", "nonmono"),
    (1, 2, 1, 128, 320, 5, 4, False, "bf16", "nonmono"),
    (1, 8, 2, 128, 256, 4, 1, True, "bf16", "beyond"),
    (1, 2, 1, 64, 128, 4, 1, True, "f32", "packed"),
    (2, 3, 1, 24, 72, 3, 0, False, "f32", "packed"),
    (1, 2, 2, 96, 128, 4, 3, True, "f32", "nonmono"),
    (1, 4, 1, 128, 160, 2, 0, True, "f32", "beyond"),
    (1, 8, 2, 128, 256, 4, 1, True, "bf16", "extreme"),
    (1, 4, 1, 128, 192, 3, 2, False, "bf16", "extreme"),
    (1, 2, 1, 64, 128, 4, 2, True, "f32", "extreme"),
]


@pytest.mark.parametrize("B,hq,hkv,d,n,c,rank,zigzag,dtype,layout", CASES)
def test_document_mask_parity(B, hq, hkv, d, n, c, rank, zigzag, dtype, layout):
    say(f"doc mask {layout} B={B} hq={hq} hkv={hkv} d={d} n={n} c={c} rank={rank} zigzag={zigzag} {dtype}")
    seed = 900 + n + c + rank
    q = random_array((B, hq, n, d), dtype, seed)
    k = random_array((c, B, hkv, n, d), dtype, seed + 1)
    v = random_array((c, B, hkv, n, d), dtype, seed + 2)
    ds = _layout(layout, c * n, seed)
    out, lse = run_gpu_doc(q, k, v, ds, c, rank, zigzag, dtype=dtype)
    ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, True, zigzag, doc_start=ds)
    assert_parity(out, ref, lse, ref_lse, dtype, f"doc {layout}")


@pytest.mark.parametrize("zigzag", [False, True])
def test_document_mask_round_ranges(zigzag):
    c, n, rank = 4, 256, 2
    q = random_array((1, 4, n, 128), "bf16", 71)
    k = random_array((c, 1, 2, n, 128), "bf16", 72)
    v = random_array((c, 1, 2, n, 128), "bf16", 73)
    ds = _layout("packed", c * n, 74)
    for t0, t1 in [(0, 1), (1, 3), (3, 4), (2, 2)]:
        say(f"doc rounds [{t0},{t1}) zigzag={zigzag}")
        out, lse = run_gpu_doc(q, k, v, ds, c, rank, zigzag, t0, t1)
        ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, True, zigzag, t0, t1, doc_start=ds)
        assert_parity(out, ref, lse, ref_lse, "bf16", f"doc rounds [{t0},{t1})")


@pytest.fixture(scope="module")
def docs_workload():
    w = WORKLOADS["gqa64x8_d128_s128k_c16_zigzag_docs_bf16"]
    say(f"generating {w.name}")
    return w, make_inputs(w), make_doc_start(w)


def test_docs_fullsize_sampled_rows(docs_workload):
    w, (q, k, v), ds = docs_workload
    n = w.rows
    say(f"{w.name}: GPU fused launch")
    out, lse = run_gpu_doc(q, k, v, ds, w.c, w.rank, w.zigzag)
    rng = np.random.default_rng(5)
    pos = oracle.chunk_positions(w.rank, n, w.c, w.zigzag)
    # rows at document starts and ends, chunk edges and at random
    starts = np.nonzero(ds[pos] == pos)[0]
    ends = np.nonzero(np.r_[ds[pos[1:]] != ds[pos[:-1]], True])[0]
    ts = np.unique(np.concatenate([starts[:20], ends[:20], [0, 1, n // 2 - 1, n // 2, n - 1],
                                   rng.integers(0, n, 60)]))
    heads = [0, 7, 8, 63]
    rows = np.array([(0, h, t) for h in heads for t in ts], dtype=np.int64)
    say(f"{w.name}: oracle on {len(rows)} rows")
    ref, ref_lse = oracle.rank_forward(q, k, v, w.c, w.rank, True, w.zigzag, rows=rows, doc_start=ds)
    got = out[rows[:, 0], rows[:, 1], rows[:, 2]]
    got_lse = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    mx, mean = assert_parity(got, ref, got_lse, ref_lse, "bf16", w.name)
    say(f"{w.name}: max abs {mx:.2e} mean abs {mean:.2e} rel-L2 {rel_l2(got, ref):.2e}")
    assert rel_l2(got, ref) < 1e-2


def test_docs_fullsize_zero_queries(docs_workload):
    """Q = 0: uniform weights over [doc_start[p], p], so lse = ln(p - doc_start[p] + 1)
    and out = the mean of those V rows (prefix sums in global order)."""
    w, (q, k, v), ds = docs_workload
    n = w.rows
    say(f"{w.name}: Q = 0 pin")
    out, lse = run_gpu_doc(np.zeros_like(q), k, v, ds, w.c, w.rank, w.zigzag)
    S = w.c * n
    pos = oracle.chunk_positions(w.rank, n, w.c, w.zigzag)
    lo = ds[pos].astype(np.int64)
    assert np.abs(lse - np.log(pos - lo + 1.0)[None, None, :]).max() <= 1e-3
    G = w.hq // w.hkv
    worst, total, cnt = 0.0, 0.0, 0
    for g in range(w.hkv):
        vg = np.zeros((S, w.head_dim))
        for j in range(w.c):
            vg[oracle.chunk_positions(j, n, w.c, w.zigzag)] = v[j, 0, g]
        cs = np.concatenate([np.zeros((1, w.head_dim)), np.cumsum(vg, axis=0)])
        mean = (cs[pos + 1] - cs[lo]) / (pos - lo + 1.0)[:, None]
        for h in range(g * G, (g + 1) * G):
            e = np.abs(out[0, h] - mean)
            worst = max(worst, float(e.max()))
            total += float(e.sum())
            cnt += e.size
    say(f"{w.name}: Q=0 max abs {worst:.2e} mean abs {total / cnt:.2e}")
    assert worst <= 2e-2 and total / cnt <= 2e-3


def test_docs_fullsize_streamed_sampled_rows(docs_workload):
    """The packed-document share streamed round by round (one ra_rank_forward_accumulate
    launch per ring round with the document mask, into an fp32 running output that starts
    at lse = -inf over NaN), rounded to bf16 at the end: sampled rows against the oracle
    and, over every row, the lse of the fused launch."""
    import torch
    import blockwise_ring_attention_amd as ra
    w, (q, k, v), ds = docs_workload
    n = w.rows
    say(f"{w.name}: streamed ring with documents, {w.c} launches")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    dd = torch.from_numpy(np.ascontiguousarray(ds, dtype=np.int32)).cuda()
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(qd.shape[:3], float("-inf"), dtype=torch.float32, device="cuda")
    for t in range(w.c):
        ra.rank_forward_accumulate(qd, kd, vd, out, lse, w.c, w.rank, True, w.zigzag, t, t + 1, doc_start=dd)
    fused_out, fused_lse = ra.rank_forward_doc(qd, kd, vd, dd, w.c, w.rank, w.zigzag)
    torch.cuda.synchronize()
    o = out.to(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    fl = fused_lse.cpu().numpy().astype(np.float64)
    del qd, kd, vd, dd, out, lse, fused_out, fused_lse
    torch.cuda.empty_cache()
    assert np.array_equal(np.isneginf(l), np.isneginf(fl))
    fin = ~np.isneginf(fl)
    assert np.abs(l[fin] - fl[fin]).max() <= 1e-3
    rng = np.random.default_rng(6)
    pos = oracle.chunk_positions(w.rank, n, w.c, w.zigzag)
    starts = np.nonzero(ds[pos] == pos)[0]
    ts = np.unique(np.concatenate([starts[:10], [0, n // 2 - 1, n // 2, n - 1], rng.integers(0, n, 40)]))
    rows = np.array([(0, h, t) for h in (0, 9, 63) for t in ts], dtype=np.int64)
    say(f"{w.name}: oracle on {len(rows)} rows")
    ref, ref_lse = oracle.rank_forward(q, k, v, w.c, w.rank, True, w.zigzag, rows=rows, doc_start=ds)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    got_lse = l[rows[:, 0], rows[:, 1], rows[:, 2]]
    mx, mean = assert_parity(got, ref, got_lse, ref_lse, "bf16", f"{w.name} streamed")
    say(f"{w.name}: streamed max abs {mx:.2e} mean abs {mean:.2e}")
