"""GPU parity of the streamed ring (ra_rank_forward_accumulate, through the C ABI): a rank
folds each arriving block into its running (out, lse) as the ring turns, and after the
last round holds the result over the whole ring ("What do you do about long sequences and
sparse models?", section "How does attention survive being split?").

Checked against the fp64 oracle's full-ring result: one launch per round in ring order,
rounds in uneven groups, rounds in reverse order (the fold is exact in any order), with
and without the document mask, both dtypes. The accumulator starts as lse = -inf with
out holding NaN, which must not reach the result. An empty round range leaves (out, lse)
bit-identical, and one fold equals ra_merge of the accumulator with the same rounds'
ra_rank_forward result."""

import numpy as np
import pytest

import oracle
from blockwise_ring_attention_amd.inputs import doc_start_from_lengths, draw_document_lengths, random_array
from tests.gpu_util import assert_parity, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # B, hq, hkv, d, n, c, rank, causal, zigzag, dtype, doc
    (1, 8, 1, 128, 512, 4, 1, True, True, "bf16", False),
    (1, 8, 2, 128, 256, 4, 0, True, False, "bf16", False),   # rank 0: rounds 1.. see no keys
    (1, 8, 2, 128, 256, 4, 3, True, False, "bf16", False),
    (2, 4, 2, 64, 136, 3, 2, False, False, "bf16", False),   # non-causal, ragged tiles
    (1, 16, 1, 128, 96, 2, 1, True, True, "bf16", False),    # two head sets
    (1, 8, 2, 128, 512, 4, 2, True, True, "bf16", True),
    (1, 4, 1, 128, 200, 3, 0, True, True, "bf16", True),     # ragged chunks (m = 100)
    (1, 2, 1, 64, 128, 4, 3, True, True, "f32", False),
    (2, 3, 1, 24, 72, 3, 0, True, False, "f32", False),
    (1, 2, 2, 96, 128, 4, 1, True, True, "f32", True),
]

GROUPINGS = {
    "per_round": lambda c: [(t, t + 1) for t in range(c)],
    "grouped": lambda c: [(0, 1), (1, c - 1), (c - 1, c)] if c > 2 else [(0, 1), (1, c)],
    "reverse": lambda c: [(t, t + 1) for t in reversed(range(c))],
}


def _inputs(B, hq, hkv, d, n, c, dtype, doc, seed):
    q = random_array((B, hq, n, d), dtype, seed)
    k = random_array((c, B, hkv, n, d), dtype, seed + 1)
    v = random_array((c, B, hkv, n, d), dtype, seed + 2)
    ds = doc_start_from_lengths(draw_document_lengths(c * n, 37, 1.2, seed)) if doc else None
    return q, k, v, ds


def _device(q, k, v, ds, dtype):
    import torch
    dd = torch.from_numpy(np.ascontiguousarray(ds, dtype=np.int32)).cuda() if ds is not None else None
    return to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), dd


def _fresh_accumulator(qd, out_f32=False):
    import torch
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32 if out_f32 else qd.dtype, device=qd.device)
    lse = torch.full(qd.shape[:3], float("-inf"), dtype=torch.float32, device=qd.device)
    return out, lse


def _host(out, lse):
    import torch
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


# bf16 inputs run with a bf16 and with an fp32 running output; fp32 inputs have only fp32
CASES_OUT = [case + (False,) for case in CASES] + [case + (True,) for case in CASES if case[9] == "bf16"]


@pytest.mark.parametrize("grouping", sorted(GROUPINGS))
@pytest.mark.parametrize("B,hq,hkv,d,n,c,rank,causal,zigzag,dtype,doc,out32", CASES_OUT)
def test_streamed_ring_parity(B, hq, hkv, d, n, c, rank, causal, zigzag, dtype, doc, out32, grouping):
    import blockwise_ring_attention_amd as ra
    say(f"accumulate {grouping} B={B} hq={hq} hkv={hkv} d={d} n={n} c={c} rank={rank} causal={causal} "
        f"zigzag={zigzag} {dtype} doc={doc} out32={out32}")
    q, k, v, ds = _inputs(B, hq, hkv, d, n, c, dtype, doc, 1300 + n + c + rank)
    qd, kd, vd, dd = _device(q, k, v, ds, dtype)
    out, lse = _fresh_accumulator(qd, out32)
    for t0, t1 in GROUPINGS[grouping](c):
        ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, rank, causal, zigzag, t0, t1, doc_start=dd)
    o, l = _host(out, lse)
    ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, causal, zigzag, doc_start=ds)
    assert_parity(o, ref, l, ref_lse, dtype, f"accumulate {grouping}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_round_range_leaves_accumulator(dtype):
    import torch
    import blockwise_ring_attention_amd as ra
    c, n, rank = 4, 256, 1
    q, k, v, _ = _inputs(1, 4, 2, 128 if dtype == "bf16" else 64, n, c, dtype, False, 41)
    qd, kd, vd, _ = _device(q, k, v, None, dtype)
    out, lse = _fresh_accumulator(qd)
    ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, rank, True, True, 0, 2)
    before_out, before_lse = out.clone(), lse.clone()
    ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, rank, True, True, 2, 2)
    torch.cuda.synchronize()
    assert torch.equal(out, before_out) and torch.equal(lse, before_lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_equals_merge_of_partials(dtype):
    """One accumulate call over rounds [2, c) == ra_merge(accumulator, ra_rank_forward over
    [2, c)): the kernel's epilogue and the merge kernel take the same combination."""
    import torch
    import blockwise_ring_attention_amd as ra
    c, n, rank, d = 4, 384, 2, 128 if dtype == "bf16" else 64
    q, k, v, _ = _inputs(1, 8, 2, d, n, c, dtype, False, 57)
    qd, kd, vd, _ = _device(q, k, v, None, dtype)
    out, lse = _fresh_accumulator(qd)
    ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, rank, True, True, 0, 2)
    acc_out, acc_lse = out.clone(), lse.clone()
    ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, rank, True, True, 2, c)
    part_out, part_lse = ra.rank_forward(qd, kd, vd, c, rank, True, True, 2, c)
    m_out, m_lse = ra.merge(acc_out, acc_lse, part_out, part_lse)
    torch.cuda.synchronize()
    diff = (out.float() - m_out.float()).abs().max().item()
    # bf16: the merge rounds the partial to bf16 before combining, the fold does not, so
    # the two may differ by about one bf16 step (2^-7 relative) of the output values.
    scale = max(1.0, m_out.float().abs().max().item())
    assert diff <= (2.0 ** -6 * scale if dtype == "bf16" else 1e-6), diff
    assert torch.allclose(lse, m_lse, rtol=0, atol=1e-5)


@pytest.mark.parametrize("out32", [False, True])
def test_streamed_ring_full_size_32k(out32):
    """The 32k GQA share (c = 8, rank 3, zigzag) streamed round by round at full size:
    equal to the fused launch within the bf16 bar, and sampled rows equal to the oracle."""
    import torch
    import blockwise_ring_attention_amd as ra
    from blockwise_ring_attention_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS["gqa32x8_d128_s32k_c8_zigzag_bf16"]
    say(f"accumulate full size {w.name}")
    q, k, v = make_inputs(w)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    fused, fused_lse = ra.rank_forward(qd, kd, vd, w.c, w.rank, w.causal, w.zigzag)
    out, lse = _fresh_accumulator(qd, out32)
    for t in range(w.c):
        ra.rank_forward_accumulate(qd, kd, vd, out, lse, w.c, w.rank, w.causal, w.zigzag, t, t + 1)
    torch.cuda.synchronize()
    diff = (out.float() - fused.float()).abs()
    assert diff.max().item() <= 2e-2 and diff.mean().item() <= 2e-3, (diff.max().item(), diff.mean().item())
    assert (lse - fused_lse).abs().max().item() <= 1e-3
    rng = np.random.default_rng(5)
    n = w.rows
    rows = np.array(sorted({(0, int(h), int(t)) for h, t in zip(rng.integers(0, w.hq, 48), rng.integers(0, n, 48))}
                           | {(0, 0, 0), (0, w.hq - 1, n - 1), (0, 5, n // 2), (0, 9, n // 2 - 1)}), dtype=np.int64)
    o, l = _host(out, lse)
    ref, ref_lse = oracle.rank_forward(q, k, v, w.c, w.rank, w.causal, w.zigzag, rows=rows)
    assert_parity(o[rows[:, 0], rows[:, 1], rows[:, 2]], ref, l[rows[:, 0], rows[:, 1], rows[:, 2]], ref_lse, "bf16",
                  "accumulate 32k sampled rows")


def test_streamed_ring_replays_in_a_graph():
    """The streamed ring captured in a HIP graph (torch.cuda.CUDAGraph): a fill of the
    running lse with -inf and one ra_rank_forward_accumulate launch per round. The library
    allocates nothing and synchronizes nothing, so the captured sequence replays; every
    replay, with unrelated eager work between replays, equals the eager run bit for bit."""
    import torch
    import blockwise_ring_attention_amd as ra
    B, hq, hkv, d, n, c, rank = 1, 8, 2, 128, 512, 4, 1
    say("streamed ring in a graph")
    q, k, v, _ = _inputs(B, hq, hkv, d, n, c, "bf16", False, 77)
    qd, kd, vd, _ = _device(q, k, v, None, "bf16")
    eager_out, eager_lse = _fresh_accumulator(qd, out_f32=True)
    for t in range(c):
        ra.rank_forward_accumulate(qd, kd, vd, eager_out, eager_lse, c, rank, True, True, t, t + 1)
    torch.cuda.synchronize()
    out = torch.empty(qd.shape, dtype=torch.float32, device=qd.device)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=qd.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm up on a side stream before capture
        lse.fill_(float("-inf"))
        for t in range(c):
            ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, rank, True, True, t, t + 1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lse.fill_(float("-inf"))
        for t in range(c):
            ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, rank, True, True, t, t + 1)
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse), f"replay {rep}"
        other, _ = ra.rank_forward(qd, kd, vd, c, rank, True, True)   # eager work between replays
        torch.cuda.synchronize()
    ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, True, True)
    o, l = _host(out, lse)
    assert_parity(o, ref, l, ref_lse, "bf16", "graph replay")
