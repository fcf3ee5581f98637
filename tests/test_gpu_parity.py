"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle, element by
element, at sizes the oracle finishes in seconds: several query and key tiles, ragged
tails, every mask mode, GQA groupings, round ranges, the merge, and edge cases."""

import numpy as np
import pytest

import oracle
from blockwise_ring_attention_amd.inputs import WORKLOADS, make_inputs, random_array
from tests.gpu_util import assert_parity, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, hq, hkv, d, nq, nkv, c, dtype, seed, scale=1.0):
    q = random_array((B, hq, nq, d), dtype, seed, scale)
    k = random_array((c, B, hkv, nkv, d), dtype, seed + 1, scale)
    v = random_array((c, B, hkv, nkv, d), dtype, seed + 2, scale)
    return q, k, v


CASES = [
    # B, hq, hkv, d, n, c, rank, causal, zigzag, dtype
    (1, 4, 1, 128, 200, 3, 1, True, True, "bf16"),      # ragged chunks (m = 100), G = 4
    (2, 6, 2, 64, 136, 4, 2, True, False, "bf16"),      # G = 3 (one head per workgroup), d = 64
    (1, 16, 1, 128, 96, 2, 1, True, True, "bf16"),      # G = 16: two head sets
    (1, 8, 1, 128, 512, 4, 0, True, True, "bf16"),      # G = 8, rank 0
    (1, 8, 2, 128, 512, 4, 3, True, True, "bf16"),      # last rank
    (1, 2, 2, 128, 320, 5, 4, True, False, "bf16"),     # contiguous causal, last rank
    (2, 4, 4, 128, 130, 3, 1, False, False, "bf16"),    # non-causal, ragged
    (1, 4, 2, 128, 256, 4, 2, False, True, "bf16"),     # zigzag without mask = non-causal
    (1, 2, 1, 64, 1000, 2, 1, True, True, "bf16"),      # odd chunk size, G = 2
    (1, 1, 1, 64, 1024, 4, 0, True, True, "f32"),
    (1, 2, 1, 8, 100, 3, 2, True, True, "f32"),
    (2, 3, 1, 24, 72, 3, 0, True, False, "f32"),
    (1, 4, 2, 40, 90, 2, 1, False, False, "f32"),
    (1, 2, 2, 96, 128, 4, 3, True, True, "f32"),
    (1, 4, 1, 128, 160, 2, 0, True, True, "f32"),
    # degenerate rings and tiny blocks
    (1, 8, 1, 128, 128, 1, 0, True, True, "bf16"),      # c = 1: no ring, zigzag chunks 0 and 1
    (1, 4, 2, 128, 100, 1, 0, True, False, "bf16"),     # c = 1, causal, ragged
    (2, 2, 1, 64, 70, 1, 0, False, False, "bf16"),      # c = 1, non-causal
    (1, 2, 1, 32, 48, 1, 0, True, True, "f32"),         # c = 1, fp32
    (1, 8, 1, 128, 2, 4, 1, True, True, "bf16"),        # one-token zigzag chunks
    (1, 4, 1, 128, 32, 3, 2, True, True, "bf16"),       # 16-token chunks, half a sub-tile
    (3, 8, 1, 128, 96, 2, 0, True, True, "bf16"),       # B x Hkv = 3: no XCD grouping
    (1, 8, 8, 128, 64, 6, 5, True, False, "bf16"),      # MHA 8 heads, last of 6 ranks, one stage
]


@pytest.mark.parametrize("B,hq,hkv,d,n,c,rank,causal,zigzag,dtype", CASES)
def test_fused_parity(B, hq, hkv, d, n, c, rank, causal, zigzag, dtype):
    say(f"fused parity B={B} hq={hq} hkv={hkv} d={d} n={n} c={c} rank={rank} causal={causal} zigzag={zigzag} {dtype}")
    q, k, v = _case(B, hq, hkv, d, n, n, c, dtype, seed=hq * 7 + n, scale=1.0)
    out, lse = run_gpu(q, k, v, c, rank, causal, zigzag, dtype=dtype)
    ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, causal, zigzag)
    assert_parity(out, ref, lse, ref_lse, dtype, "fused")


def test_noncausal_nq_differs_from_nkv():
    say("non-causal nq != nkv")
    q, k, v = _case(2, 4, 2, 128, 70, 130, 3, "bf16", seed=5)
    out, lse = run_gpu(q, k, v, 3, 2, False, False)
    ref, ref_lse = oracle.rank_forward(q, k, v, 3, 2, False, False)
    assert_parity(out, ref, lse, ref_lse, "bf16", "nq!=nkv")


def test_tiny_worked_example_fp32():
    w = WORKLOADS["tiny_c3_d8_fp32"]
    say(f"workload {w.name}")
    q, k, v = make_inputs(w)
    out, lse = run_gpu(q, k, v, w.c, w.rank, w.causal, w.zigzag, dtype="f32")
    ref, ref_lse = oracle.rank_forward(q, k, v, w.c, w.rank, w.causal, w.zigzag)
    assert_parity(out, ref, lse, ref_lse, "f32", w.name)


def test_mha_d64_s4k_zigzag_fp32_all_rows():
    w = WORKLOADS["mha_d64_s4k_c4_zigzag_fp32"]
    say(f"workload {w.name}")
    q, k, v = make_inputs(w)
    out, lse = run_gpu(q, k, v, w.c, w.rank, w.causal, w.zigzag, dtype="f32")
    ref, ref_lse = oracle.rank_forward(q, k, v, w.c, w.rank, w.causal, w.zigzag)
    assert_parity(out, ref, lse, ref_lse, "f32", w.name)


@pytest.mark.parametrize("causal,zigzag,dtype", [(True, True, "bf16"), (True, False, "bf16"),
                                                 (False, False, "bf16"), (True, True, "f32")])
def test_round_ranges_and_masked_rows(causal, zigzag, dtype):
    say(f"round ranges causal={causal} zigzag={zigzag} {dtype}")
    c, n = 4, 192
    q, k, v = _case(1, 4, 2, 128 if dtype == "bf16" else 64, n, n, c, dtype, seed=31)
    for rank in (0, 2):
        for t0, t1 in [(0, 1), (1, 2), (1, 3), (3, 4), (2, 2), (0, 4)]:
            out, lse = run_gpu(q, k, v, c, rank, causal, zigzag, t0, t1, dtype=dtype)
            ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, causal, zigzag, t0, t1)
            assert_parity(out, ref, lse, ref_lse, dtype, f"rank {rank} rounds [{t0},{t1})")


def test_per_round_plus_merge_equals_fused():
    import torch
    import blockwise_ring_attention_amd as ra
    say("per-round + merge vs fused")
    c, n, rank = 4, 256, 1
    q, k, v = _case(1, 8, 2, 128, n, n, c, "bf16", seed=41)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    fused, fl = ra.rank_forward(qd, kd, vd, c, rank, True, True)
    acc, al = ra.rank_forward(qd, kd, vd, c, rank, True, True, 0, 1)
    acc32 = acc.float()
    for t in range(1, c):
        part, pl = ra.rank_forward(qd, kd, vd, c, rank, True, True, t, t + 1)
        acc32, al = ra.merge(acc32, al, part.float(), pl, out=acc32, lse=al)   # in place, fp32 carry
    torch.cuda.synchronize()
    ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, True, True)
    assert_parity(acc32.cpu().numpy().astype(np.float64), ref, al.cpu().numpy().astype(np.float64), ref_lse,
                  "bf16", "merged rounds")
    d = np.abs(acc32.cpu().numpy() - fused.float().cpu().numpy())
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert np.abs(al.cpu().numpy() - fl.cpu().numpy()).max() <= 1e-3


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 8), ("f32", 128), ("f32", 512)])
def test_merge_parity(dtype, d):
    import torch
    import blockwise_ring_attention_amd as ra
    say(f"merge parity {dtype} d={d}")
    rows = 1000
    rng = np.random.default_rng(d)
    oa = random_array((rows, d), dtype, 1)
    ob = random_array((rows, d), dtype, 2)
    la = (rng.standard_normal(rows) * 4).astype(np.float32)
    lb = (rng.standard_normal(rows) * 4).astype(np.float32)
    la[::7] = -np.inf
    lb[::11] = -np.inf
    lb[3] = la[3] = -np.inf
    ref_o, ref_l = oracle.merge(oa, la, ob, lb)
    oad, obd = to_dev(oa, dtype), to_dev(ob, dtype)
    lad, lbd = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    o, l = ra.merge(oad, lad, obd, lbd)
    torch.cuda.synchronize()
    assert_parity(o.float().cpu().numpy().astype(np.float64), ref_o, l.cpu().numpy().astype(np.float64), ref_l,
                  dtype, "merge")
    # in place into a
    ra.merge(oad, lad, obd, lbd, out=oad, lse=lad)
    torch.cuda.synchronize()
    assert np.array_equal(oad.float().cpu().numpy(), o.float().cpu().numpy())
    assert np.array_equal(lad.cpu().numpy(), l.cpu().numpy())


def test_no_keys_gives_zero_and_neg_inf():
    import torch
    import blockwise_ring_attention_amd as ra
    say("nkv = 0 and empty round range")
    q = to_dev(random_array((1, 2, 40, 128), "bf16", 3), "bf16")
    k = torch.empty((2, 1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    out, lse = ra.rank_forward(q, k, k, 2, 0, False, False)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    kk = to_dev(random_array((2, 1, 2, 40, 128), "bf16", 4), "bf16")
    out, lse = ra.rank_forward(q, kk, kk, 2, 1, True, True, 1, 1)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_lse_optional_and_repeatable():
    import torch
    import blockwise_ring_attention_amd as ra
    say("lse NULL and bitwise repeatability")
    q, k, v = _case(1, 8, 1, 128, 256, 256, 4, "bf16", seed=77)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o1, l1 = ra.rank_forward(qd, kd, vd, 4, 2, True, True)
    o2, l2 = ra.rank_forward(qd, kd, vd, 4, 2, True, True, with_lse=False)
    torch.cuda.synchronize()
    assert l2 is None
    assert torch.equal(o1, o2)


def test_binding_rejects_bad_tensors():
    import torch
    import blockwise_ring_attention_amd as ra
    q = torch.zeros((1, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 1, 3, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ra.rank_forward(q, k, k, 2, 0, True, True)          # hq % hkv != 0
    with pytest.raises(ValueError):
        ra.rank_forward(q, k[:, :, :2], k[:, :, :2], 2, 0, True, True)   # not contiguous
    k2 = torch.zeros((2, 1, 2, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ra.rank_forward(torch.zeros((1, 4, 64, 96), dtype=torch.bfloat16, device="cuda"), k2, k2, 2, 0, True, True)
    # preallocated results: host lse, wrong shapes, dtypes or layouts are refused before any launch
    kk = torch.zeros((2, 1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ra.rank_forward(q, kk, kk, 2, 0, True, True, lse=torch.empty((1, 4, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        ra.rank_forward_accumulate(q, kk, kk, torch.empty_like(q), torch.empty((1, 4, 64), dtype=torch.float32),
                                   2, 0, True, True)
    with pytest.raises(ValueError):
        ra.rank_forward(q, kk, kk, 2, 0, True, True, out=torch.empty_like(q, device="cpu"))
    oa = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    la = torch.zeros((4,), dtype=torch.float32, device="cuda")
    bad_outs = [torch.empty((3, 128), dtype=torch.bfloat16, device="cuda"),     # too small
                torch.empty((4, 128), dtype=torch.float32, device="cuda"),      # other dtype
                torch.empty((4, 128), dtype=torch.bfloat16),                    # host memory
                torch.empty((128, 4), dtype=torch.bfloat16, device="cuda").t()]  # not contiguous
    for bo in bad_outs:
        with pytest.raises(ValueError):
            ra.merge(oa, la, oa, la, out=bo)
    bad_lses = [torch.empty((3,), dtype=torch.float32, device="cuda"),
                torch.empty((4,), dtype=torch.bfloat16, device="cuda"),
                torch.empty((4,), dtype=torch.float32)]
    for bl in bad_lses:
        with pytest.raises(ValueError):
            ra.merge(oa, la, oa, la, lse=bl)
    with pytest.raises(ValueError):
        ra.merge(oa, la.cpu(), oa, la)


def test_causal_mask_regression_inputs():
    """Plain causal zigzag on the inputs that exposed a miscompiled mask: written with
    short-circuit operators and an if, the compiler's lowering of the per-key mask lost
    the masking store for some lanes whenever a query tile's diagonal fell in the first
    32 keys of a stage (every query then saw up to 31 later keys)."""
    B, hq, hkv, d, n, c, rank = 1, 8, 1, 128, 512, 4, 0
    seed = 900 + n + c + rank
    q = random_array((B, hq, n, d), "bf16", seed)
    k = random_array((c, B, hkv, n, d), "bf16", seed + 1)
    v = random_array((c, B, hkv, n, d), "bf16", seed + 2)
    for zigzag in (True, False):
        say(f"mask regression zigzag={zigzag}")
        out, lse = run_gpu(q, k, v, c, rank, True, zigzag)
        ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, True, zigzag)
        assert_parity(out, ref, lse, ref_lse, "bf16", "mask regression")


@pytest.mark.parametrize("pattern", ["large", "rising", "falling"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reference_raise_paths(pattern, dtype):
    """Scores that keep the online softmax's reference moving: large-magnitude Q/K
    (scaled scores in the hundreds, so the running maximum jumps far and often), keys
    whose scores rise along the sequence (a new maximum at every sub-tile) and fall
    along it (the first sub-tile holds the maximum). The fp64 oracle has no reference
    at all, so any slip in the rescaling shows up here."""
    B, hq, hkv, d, n, c, rank = 1, 4, 2, (128 if dtype == "bf16" else 64), 256, 4, 1
    seed = 4100 + (0 if dtype == "bf16" else 7)
    q = random_array((B, hq, n, d), dtype, seed)
    k = random_array((c, B, hkv, n, d), dtype, seed + 1)
    v = random_array((c, B, hkv, n, d), dtype, seed + 2)
    if pattern == "large":
        q = random_array((B, hq, n, d), dtype, seed, scale=6.0)
        k = random_array((c, B, hkv, n, d), dtype, seed + 1, scale=6.0)
    else:
        # a common direction in every query, and keys whose component along it follows the
        # key's global position (rising) or its negative (falling): the scaled score moves
        # by about 10 (log2 units) per 32 keys, past the reference's slack of 8 each time
        q = q.copy()
        q[..., 0] += 16.0
        pos = np.stack([oracle.chunk_positions(j, n, c, True) for j in range(c)])   # [c, n]
        sign = 1.0 if pattern == "rising" else -1.0
        k = k.copy()
        k[..., 0] = (sign * 155.0 * pos / (c * n))[:, None, None, :]
        from blockwise_ring_attention_amd.inputs import round_to_dtype
        q, k = round_to_dtype(q, dtype), round_to_dtype(k, dtype)
    # fp32 rounding of a score grows with the size of its terms: the fp32 bar (1e-5, for
    # scores of order 1) is scaled by the largest |score| over 4, bf16 keeps its bar
    kall = k.reshape(c, B, hkv, n, d).transpose(1, 2, 0, 3, 4).reshape(B, hkv, c * n, d).astype(np.float64)
    smax = max(float(np.abs(q[0, h].astype(np.float64) @ kall[0, h // (hq // hkv)].T).max()) for h in range(hq))
    smax /= np.sqrt(d)
    for causal in (True, False):
        say(f"reference raise {pattern} {dtype} causal={causal} max|score| {smax:.1f}")
        out, lse = run_gpu(q, k, v, c, rank, causal, True, dtype=dtype)
        ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, causal, True)
        if dtype == "bf16":
            assert_parity(out, ref, lse, ref_lse, dtype, f"reference raise {pattern}")
        else:
            tol = 1e-5 * max(1.0, smax / 4.0)
            err = np.abs(out - ref).max()
            assert np.all(np.isfinite(out)) and err <= tol, (err, tol)
            assert np.abs(lse - ref_lse).max() <= 1e-3


def test_concurrent_streams_give_the_same_result():
    """The library keeps no device state between or across calls: launches of different
    problems on two streams at once (default priority) give bit-identical results to the
    same launches one after the other."""
    import torch
    import blockwise_ring_attention_amd as ra
    say("two streams at once")
    cases = [(1, 8, 2, 128, 512, 4, 1, True, True), (2, 4, 4, 64, 264, 3, 0, False, False)]
    inputs = []
    for i, (B, hq, hkv, d, n, c, rank, causal, zigzag) in enumerate(cases):
        q, k, v = _case(B, hq, hkv, d, n, n, c, "bf16", seed=5100 + 17 * i)
        inputs.append((to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), c, rank, causal, zigzag))
    alone = []
    for qd, kd, vd, c, rank, causal, zigzag in inputs:
        out, lse = ra.rank_forward(qd, kd, vd, c, rank, causal, zigzag)
        torch.cuda.synchronize()
        alone.append((out.clone(), lse.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    together = []
    for rep in range(3):
        res = []
        for s, (qd, kd, vd, c, rank, causal, zigzag) in zip(streams, inputs):
            with torch.cuda.stream(s):
                res.append(ra.rank_forward(qd, kd, vd, c, rank, causal, zigzag))
        torch.cuda.synchronize()
        together.append(res)
    for res in together:
        for (out, lse), (out0, lse0) in zip(res, alone):
            assert torch.equal(out, out0) and torch.equal(lse, lse0)


@pytest.mark.parametrize("c,rank,n,causal,zigzag,doc", [
    (32, 0, 64, True, True, False), (32, 31, 66, True, True, False), (64, 17, 32, True, False, False),
    (64, 40, 130, True, True, True), (48, 5, 40, False, False, False),
])
def test_long_rings(c, rank, n, causal, zigzag, doc):
    """Rings of 32 to 64 ranks with short blocks: the cursor walks many rounds and
    segments per tile (most empty under the causal and document masks), fused and folded
    round by round into an fp32 running output."""
    import torch
    import blockwise_ring_attention_amd as ra
    from blockwise_ring_attention_amd.inputs import doc_start_from_lengths, draw_document_lengths
    say(f"long ring c={c} rank={rank} n={n} causal={causal} zigzag={zigzag} doc={doc}")
    q, k, v = _case(1, 8, 2, 128, n, n, c, "bf16", seed=6100 + c + rank)
    ds = doc_start_from_lengths(draw_document_lengths(c * n, 300, 1.0, c + rank)) if doc else None
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    dd = torch.from_numpy(np.ascontiguousarray(ds, dtype=np.int32)).cuda() if doc else None
    if doc:
        out, lse = ra.rank_forward_doc(qd, kd, vd, dd, c, rank, zigzag)
    else:
        out, lse = ra.rank_forward(qd, kd, vd, c, rank, causal, zigzag)
    acc = torch.empty(qd.shape, dtype=torch.float32, device=qd.device)
    acc_lse = torch.full(qd.shape[:3], float("-inf"), device=qd.device)
    for t in range(c):
        ra.rank_forward_accumulate(qd, kd, vd, acc, acc_lse, c, rank, causal, zigzag, t, t + 1, doc_start=dd)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, causal, zigzag, doc_start=ds)
    assert_parity(out.float().cpu().numpy().astype(np.float64), ref, lse.cpu().numpy().astype(np.float64), ref_lse,
                  "bf16", "fused")
    assert_parity(acc.cpu().numpy().astype(np.float64), ref, acc_lse.cpu().numpy().astype(np.float64), ref_lse,
                  "bf16", "streamed")
