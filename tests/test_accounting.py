"""Closed-form work/traffic counts (host logic used by the bench) pinned against the
oracle's brute-force counts and against the figures the pages print."""

import json
import os

import numpy as np
import pytest

from blockwise_ring_attention_amd import accounting as acc
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("zigzag", [False, True])
def test_allowed_entries_match_bruteforce(zigzag):
    for c in range(1, 9):
        for m in range(1, 8):
            rows = 2 * m if zigzag else m
            for rank in range(c):
                brute = A.allowed_count(c, rank, rows, True, zigzag)
                assert acc.allowed_entries(c, rank, rows, rows, True, zigzag) == brute
                for t in range(c):
                    assert acc.allowed_entries(c, rank, rows, rows, True, zigzag, t, t + 1) == \
                        A.allowed_count(c, rank, rows, True, zigzag, t, t + 1)


def test_zigzag_closed_form_equal_for_every_rank():
    for c in range(1, 9):
        for m in range(1, 8):
            counts = {A.allowed_count(c, r, 2 * m, True, True) for r in range(c)}
            assert counts == {(2 * c - 1) * m * m + m * (m + 1)}


def test_load_balance_units_from_the_page():
    g = json.load(open(os.path.join(GOLDEN, "load_balance.json")))
    c = g["c"]
    contiguous = [A.chunk_units(c, r, False) for r in range(c)]
    assert contiguous == g["contiguous_units"]
    assert max(contiguous) // min(contiguous) == g["contiguous_spread"]
    assert all(A.chunk_units(c, r, True) == g["zigzag_units_per_rank"] for r in range(c))
    for cc in range(1, 12):
        assert all(A.chunk_units(cc, r, True) == 2 * cc + 1 for r in range(cc))
        assert [A.chunk_units(cc, r, False) for r in range(cc)] == list(range(1, cc + 1))


def test_needed_rows_match_bruteforce():
    import numpy as np
    for zigzag in (False, True):
        for c in range(1, 7):
            for m in (1, 3, 4):
                rows = 2 * m if zigzag else m
                for rank in range(c):
                    pq = A.chunk_positions(rank, rows, c, zigzag)
                    for j in range(c):
                        pk = A.chunk_positions(j, rows, c, zigzag)
                        brute = int(A.causal_allowed(pq, pk).any(axis=0).sum())
                        assert acc.needed_kv_rows(c, rank, j, rows, True, zigzag) == brute
                        assert acc.needed_kv_rows(c, rank, j, rows, False, zigzag) == rows
    assert np.isfinite(1.0)


def test_flop_convention_against_page():
    g = json.load(open(os.path.join(GOLDEN, "attention_flops.json")))
    S, L, h = g["seq"], g["layers"], g["hidden"]
    # full rows, one layer, one head of width h: forward = 4 h S^2; fwd + bwd = 3x
    fwd = acc.unmasked_flop(1, 1, h, acc.allowed_entries(1, 0, S, S, False, False))
    per_token = 3 * L * fwd / S
    assert round(per_token / 1e9) == g["gflop_per_token"]


def test_break_even_figures_from_the_page():
    g = json.load(open(os.path.join(GOLDEN, "ring_break_even.json")))
    t = acc.ring_break_even_tokens(g["flops_per_s"], g["nvlink_bytes_per_s"])
    assert round(t) == g["nvlink_tokens_per_block"]
    assert round(6 * t, -3) == g["nvlink_tokens_per_rank_about"]
    tp = acc.ring_break_even_tokens(g["flops_per_s"], g["port_bits_per_s"] / 8)
    assert round(tp) == g["port_tokens_per_block"]
    assert round(g["blocks_per_sequence"] * tp, -3) == g["port_tokens_per_rank_about"]


def test_workload_flops_and_bytes():
    from blockwise_ring_attention_amd.inputs import WORKLOADS
    w = WORKLOADS["gqa64x8_d128_s128k_c16_zigzag_bf16"]
    n = w.rows
    e = acc.allowed_entries(w.c, w.rank, n, n, True, True)
    assert e == 536_875_008
    assert acc.unmasked_flop(w.batch, w.hq, w.head_dim, e) == 4 * 128 * e * 64
    w3 = WORKLOADS["gqa32x8_d128_s32k_c8_zigzag_bf16"]
    e3 = acc.allowed_entries(w3.c, w3.rank, w3.rows, w3.rows, True, True)
    assert e3 == 67_110_912


def test_document_counts_match_brute_force():
    """The closed-form document-mask counts used by the bench equal the oracle's
    brute-force counts (allowed entries) and a direct union of visible key positions."""
    import numpy as np
    import oracle
    from blockwise_ring_attention_amd import accounting as acc
    from blockwise_ring_attention_amd.inputs import doc_start_from_lengths, draw_document_lengths
    c, rows = 4, 32
    S = c * rows
    for seed, layout in enumerate([draw_document_lengths(S, 9, 1.0, 3), [S], [1] * S]):
        ds = doc_start_from_lengths(layout)
        for zigzag in (False, True):
            for r in range(c):
                assert acc.doc_allowed_entries(c, r, rows, zigzag, ds) == \
                    oracle.allowed_count(c, r, rows, True, zigzag, doc_start=ds)
                pos = oracle.chunk_positions(r, rows, c, zigzag)
                seen = set()
                for p in pos:
                    seen.update(range(int(ds[p]), int(p) + 1))
                assert acc.doc_needed_kv_rows(c, r, rows, zigzag, ds) == len(seen)
    # a start past the query leaves the row empty
    ds = np.arange(S, dtype=np.int32) + 1
    assert acc.doc_allowed_entries(c, 1, rows, True, ds) == 0
    assert acc.doc_needed_kv_rows(c, 1, rows, True, ds) == 0


def test_binding_rejects_host_doc_start():
    import pytest
    import torch
    import blockwise_ring_attention_amd as ra
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(2, 1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="doc_start"):
        ra.rank_forward_doc(q, k, k, torch.zeros(8, dtype=torch.int32), 2, 0, True)


@pytest.mark.parametrize("name", ["mha_d64_s4k_c4_zigzag_fp32", "gqa64x8_d128_s128k_c16_zigzag_bf16",
                                  "gqa64x8_d128_s128k_c16_zigzag_docs_bf16", "tiny_c3_d8_fp32"])
def test_cpu_sample_counts_its_rows(name):
    """The CPU baseline's sample: rows spread over the share, and its FLOP count equal to
    the oracle's allowed-key count of exactly those rows."""
    import bench
    from blockwise_ring_attention_amd.inputs import WORKLOADS, make_doc_start
    w = WORKLOADS[name]
    rows, flop = bench.cpu_sample(w, 96)
    n = w.rows
    assert len(rows) == min(96, w.hq * n) and (rows[:, 0] == 0).all()
    assert len({tuple(r) for r in rows}) == len(rows)
    if w.hq * n >= 192:   # both halves of a zigzag share are represented
        assert (rows[:, 2] < n // 2).any() and (rows[:, 2] >= n // 2).any()
    ds = make_doc_start(w)
    if not w.causal:
        allowed = len(rows) * n * w.c
    else:
        pq = A.chunk_positions(w.rank, n, w.c, w.zigzag)[rows[:, 2]]
        pk = np.concatenate([A.chunk_positions(j, n, w.c, w.zigzag) for j in range(w.c)])
        m = A.causal_allowed(pq, pk) if ds is None else A.document_allowed(pq, pk, ds)
        allowed = int(m.sum())
    assert flop == 4 * w.head_dim * allowed


def test_bench_break_even_context():
    """The bench line's ring arithmetic: the pages' H100 figure ("What do you do about long
    sequences and sparse models?", section "When is the ring actually free?", the golden
    fixture), the same c >= F / B with this GPU's peak and one xGMI link, and for the
    zigzag GQA share a non-local round's share of the launch, 2 m^2 of its (2c-1) m^2 +
    m(m+1) allowed entries per head."""
    import bench
    from blockwise_ring_attention_amd.inputs import WORKLOADS
    g = json.load(open(os.path.join(GOLDEN, "ring_break_even.json")))
    w = WORKLOADS["gqa64x8_d128_s128k_c16_zigzag_bf16"]
    ctx = bench.break_even_context(w, kernel_ms=14.0, tflops=1250.0)
    assert round(ctx["pages_break_even_tokens"]) == g["nvlink_tokens_per_block"]
    assert ctx["same_arithmetic_mi355x_peak_one_xgmi_link_tokens"] == pytest.approx(2516.6e12 / 153e9, rel=1e-4)
    assert ctx["same_arithmetic_measured_rate_one_xgmi_link_tokens"] == pytest.approx(1250e12 / 153e9, rel=1e-4)
    m = w.rows // 2
    frac = 2 * m * m / ((2 * w.c - 1) * m * m + m * (m + 1))
    assert ctx["nonlocal_round_ms_at_measured_rate"] == pytest.approx(14.0 * frac, abs=1e-4)
    assert ctx["kv_block_bytes"] == 2 * w.batch * w.hkv * w.rows * w.head_dim * 2
    # m >= F Hkv / (L Hq) for the GQA share
    assert ctx["min_chunk_tokens_to_hide_on_one_link"] == pytest.approx(1250e12 * w.hkv / (153e9 * w.hq), rel=1e-4)


def test_bench_traffic_only_for_the_profiled_kernel(monkeypatch, ra_lib):
    """roofline.traffic comes from the committed counter profile only while the library
    the bench loads is the build the profile was taken on; otherwise it is null."""
    import bench
    rec = json.load(open(os.path.join(os.path.dirname(bench.__file__), "profiles",
                                      "traffic_gqa64x8_d128_s128k_c16_zigzag_bf16.json")))
    assert len(rec["library_sha"]) == 16 and len(rec["kernel_sha"]) == 16
    got = bench.measured_traffic("gqa64x8_d128_s128k_c16_zigzag_bf16", 14.0)
    if rec["library_sha"] == bench.library_sha():
        assert got == pytest.approx(rec["hbm_bytes_per_launch"])
    else:
        assert got is None
    monkeypatch.setattr(bench, "library_sha", lambda: "0" * 16)
    assert bench.measured_traffic("gqa64x8_d128_s128k_c16_zigzag_bf16", 14.0) is None


def test_bench_timeline_summary_of_a_known_recording():
    """bench.summarize_timeline on a hand-built recording (2 XCDs' worth of CUs, ticks of
    the 100 MHz clock): XCD ends, per-XCD stage time, prologue, tail, relaunch gap and
    the round-robin offset come out as constructed."""
    import bench
    rows = []
    # 16 workgroups, starting XCD 3: workgroup i on XCD (i + 3) % 8; two per XCD, both
    # on one CU of that XCD, back to back. Each: entry, +400 ticks (4 us) to the first
    # barrier, 10 stages of 170 ticks, +500 ticks (5 us) of tail, then a 250-tick gap.
    t_next = {}
    for i in range(16):
        x = (i + 3) % 8
        cu_field = 5   # same CU index on every XCD
        start = t_next.get(x, 1000 + 50 * x)
        slow = 1.0 + 0.01 * x   # XCD x runs (1 + x/100) slower
        t1 = start + 400
        t2 = t1 + int(round(10 * 170 * slow))
        t3 = t2 + 500
        t_next[x] = t3 + 250
        rows.append([start, t1, t2, t3, cu_field << 8, x, 10, (32 * i) << 16 | (i % 4)])
    rec = np.zeros((64, 8), dtype=np.int64)
    rec[:16] = np.array(rows, dtype=np.int64)
    s = bench.summarize_timeline(rec, kernel_ms=0.05)
    assert s["workgroups"] == 16 and s["cus"] == 8 and s["tiles_per_cu"] == 2.0
    assert s["xcd_offset"] == 3
    assert s["prologue_us_median"] == pytest.approx(4.0) and s["tail_us_median"] == pytest.approx(5.0)
    assert s["relaunch_gap_us_median"] == pytest.approx(2.5)
    t0 = min(r[0] for r in rows)
    for x in s["xcd"]:
        mine = [r for r in rows if r[5] == x["xcd"]]
        assert x["workgroups"] == 2 and x["cus"] == 1
        assert x["end_us"] == pytest.approx((max(r[3] for r in mine) - t0) / 100.0, abs=0.05)
        assert x["us_per_stage"] == pytest.approx(1.7 * (1.0 + 0.01 * x["xcd"]), rel=2e-3)
    ends = np.array([x["end_us"] for x in s["xcd"]])
    assert s["slowest_xcd_over_mean"] == pytest.approx(ends.max() / ends.mean() - 1, abs=1e-4)
    # a recording whose XCDs do not follow one round-robin offset reports none
    rec[1, 5] = 7
    assert bench.summarize_timeline(rec, kernel_ms=0.05)["xcd_offset"] is None
