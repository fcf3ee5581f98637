"""The design-choice comparison libraries compute what the shipped one computes.

The build script compiles one library per design-choice switch (see the top of
ra_fwd.hip): KV heads scattered over the XCDs, unswizzled LDS rows, no causal tile
skipping, one query head per workgroup, a barrier before every stage. They exist to
measure what each choice is worth, so each must give the shipped library's result:
bit-identical (every row's keys are folded in the same order with the same arithmetic;
skipped tiles would only have added exact zeros), and within the parity bar of the fp64
oracle. Called through the C ABI of each library.
"""

import ctypes
import os

import numpy as np
import pytest

import oracle
from blockwise_ring_attention_amd.inputs import random_array
from tests.gpu_util import assert_parity, say, to_dev

pytestmark = pytest.mark.gpu

NAMES = ["xcd_scatter", "no_swizzle", "no_skip", "one_head", "stage_barrier"]


def _run(lib_path, q, k, v, c, rank, causal, zigzag):
    import torch
    from blockwise_ring_attention_amd import _binding
    lib = _binding.load(lib_path)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    B, hq, nq, d = q.shape
    hkv, nkv = k.shape[2], k.shape[3]
    out = torch.empty_like(qd)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device="cuda")
    code = lib.ra_rank_forward(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(), B, hq,
                               hkv, nq, nkv, d, c, rank, int(causal), int(zigzag), 0, c, _binding.RA_BF16,
                               torch.cuda.current_stream().cuda_stream)
    assert code == 0, lib.ra_last_error()
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("causal,zigzag", [(True, True), (True, False), (False, False)])
def test_ablation_library_matches_shipped(name, causal, zigzag):
    from blockwise_ring_attention_amd import _binding
    from blockwise_ring_attention_amd.csrc import build
    path = build.ablation_path(name)
    assert os.path.exists(path), f"{path} is missing: run __graft_entry__.build()"
    # 8 KV heads (the XCD mapping applies), 2 query heads each, ragged zigzag chunks
    B, hq, hkv, d, n, c, rank = 1, 16, 8, 128, 328, 4, 2
    seed = 3100 + 7 * c + rank
    q = random_array((B, hq, n, d), "bf16", seed)
    k = random_array((c, B, hkv, n, d), "bf16", seed + 1)
    v = random_array((c, B, hkv, n, d), "bf16", seed + 2)
    say(f"ablation {name} causal={causal} zigzag={zigzag}")
    got, got_lse = _run(path, q, k, v, c, rank, causal, zigzag)
    ref_out, ref_lse_s = _run(_binding.LIB_PATH, q, k, v, c, rank, causal, zigzag)
    assert np.array_equal(got, ref_out), f"{name}: out differs from the shipped library"
    assert np.array_equal(got_lse, ref_lse_s), f"{name}: lse differs from the shipped library"
    ref, ref_lse = oracle.rank_forward(q, k, v, c, rank, causal, zigzag)
    assert_parity(got.astype(np.float64), ref, got_lse.astype(np.float64), ref_lse, "bf16", name)
