"""GPU parity at every stage count from 1 to 6 (through the C ABI).

The bf16 kernel folds its 64-key stages in pairs, with one workgroup barrier per pair; a
fold that ends on an odd stage waits for that stage's V tile with one more barrier before
its tail, and one that ends on an even stage does not. In a non-causal launch over one
block every tile folds the same number of stages, ceil(nkv / 64), so each count here
drives every tile of the launch down one of the two endings (1: the first stage only).
Fused, and streamed one round at a time into bf16 and fp32 running outputs, against the
fp64 oracle."""

import pytest

import oracle
from blockwise_ring_attention_amd.inputs import random_array
from tests.gpu_util import assert_parity, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu

STAGES = [1, 2, 3, 4, 5, 6]


def _inputs(d, nkv, c, seed, nq=96, hq=8, hkv=2):
    q = random_array((1, hq, nq, d), "bf16", seed)
    k = random_array((c, 1, hkv, nkv, d), "bf16", seed + 1)
    v = random_array((c, 1, hkv, nkv, d), "bf16", seed + 2)
    return q, k, v


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("stages", STAGES)
def test_fused_every_stage_count(d, stages):
    nkv = 64 * stages - 5   # a ragged last stage
    say(f"fused, {stages} stages per tile, d={d}, nkv={nkv}")
    q, k, v = _inputs(d, nkv, 1, 4100 + 10 * stages + d)
    out, lse = run_gpu(q, k, v, 1, 0, False, False)
    ref, ref_lse = oracle.rank_forward(q, k, v, 1, 0, False, False)
    assert_parity(out, ref, lse, ref_lse, "bf16", f"{stages} stages")


@pytest.mark.parametrize("out32", [False, True])
@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("stages", STAGES)
def test_streamed_every_stage_count(d, stages, out32):
    import numpy as np
    import torch
    import blockwise_ring_attention_amd as ra
    c, nkv = 3, 64 * stages - 5
    say(f"streamed, {stages} stages per tile and round, d={d}, nkv={nkv}, out32={out32}")
    q, k, v = _inputs(d, nkv, c, 4300 + 10 * stages + d)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32 if out32 else qd.dtype, device=qd.device)
    lse = torch.full(qd.shape[:3], float("-inf"), dtype=torch.float32, device=qd.device)
    for t in range(c):
        ra.rank_forward_accumulate(qd, kd, vd, out, lse, c, 0, False, False, t, t + 1)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    ls = lse.cpu().numpy().astype(np.float64)
    ref, ref_lse = oracle.rank_forward(q, k, v, c, 0, False, False)
    assert_parity(o, ref, ls, ref_lse, "bf16", f"streamed {stages} stages")
