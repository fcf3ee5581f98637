"""The diagnostic timeline build records its workgroups without changing the result.

The build script makes one library with per-workgroup clock stamps in the bf16 kernel
(see the top of ra_fwd.hip). It backs `bench.py --timeline`, which reads the per-XCD
finish times and the per-tile fixed costs off it, so it must give the shipped library's
result bit for bit, write only inside the registered capacity, and record stamps in
their order. Called through the C ABI of both libraries.
"""

import ctypes
import os

import numpy as np
import pytest

from blockwise_ring_attention_amd.inputs import random_array
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _lib():
    from blockwise_ring_attention_amd import _binding
    from blockwise_ring_attention_amd.csrc import build
    path = build.ablation_path("timeline")
    assert os.path.exists(path), f"{path} is missing: run __graft_entry__.build()"
    lib = _binding.load(path)
    lib.ra_diag_timeline.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.ra_diag_timeline.restype = ctypes.c_int
    return lib


def _run(lib, qd, kd, vd, c, rank):
    import torch
    from blockwise_ring_attention_amd import _binding
    B, hq, nq, d = qd.shape
    hkv, nkv = kd.shape[2], kd.shape[3]
    out = torch.empty_like(qd)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device="cuda")
    code = lib.ra_rank_forward(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(), B, hq,
                               hkv, nq, nkv, d, c, rank, 1, 1, 0, c, _binding.RA_BF16,
                               torch.cuda.current_stream().cuda_stream)
    assert code == 0, lib.ra_last_error()
    torch.cuda.synchronize()
    return out, lse


def test_timeline_records_without_changing_the_result():
    import torch
    from blockwise_ring_attention_amd import _binding
    lib = _lib()
    B, hq, hkv, d, n, c, rank = 1, 16, 8, 128, 328, 4, 2
    q = random_array((B, hq, n, d), "bf16", 4100)
    k = random_array((c, B, hkv, n, d), "bf16", 4101)
    v = random_array((c, B, hkv, n, d), "bf16", 4102)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    ref_out, ref_lse = _run(_binding.load(), qd, kd, vd, c, rank)

    cap = 1024
    buf = torch.zeros((cap + 1, 8), dtype=torch.int64, device="cuda")
    buf[cap] = -7   # a row past the capacity: must stay as it is
    torch.cuda.synchronize()
    say("timeline: full capacity")
    assert lib.ra_diag_timeline(ctypes.c_void_p(buf.data_ptr()), cap) == 0
    out, lse = _run(lib, qd, kd, vd, c, rank)
    assert lib.ra_diag_timeline(None, 0) == 0
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    rec = buf.cpu().numpy()
    assert (rec[cap] == -7).all()
    n_wg = int(np.count_nonzero(rec[:cap, 0]))
    assert n_wg > 8
    assert not rec[n_wg:cap].any(), "recorded rows are not the first workgroups"
    r = rec[:n_wg]
    folded = r[:, 1] != 0
    assert folded.any()
    assert (r[folded, 0] <= r[folded, 1]).all() and (r[folded, 1] <= r[folded, 2]).all()
    assert (r[folded, 2] <= r[folded, 3]).all() and (r[:, 0] <= r[:, 3]).all()
    # workgroups are dealt round-robin to the 8 XCDs, starting where the previous dispatch
    # left off: workgroup i runs on XCD (i + o) mod 8 with one o per launch, so workgroups
    # i and i + 8 share an XCD (what the kernel's KV-head pinning relies on)
    off = ((r[:, 5] & 0xF) - np.arange(n_wg)) % 8
    assert (off == off[0]).all(), "workgroups i and i + 8 share an XCD"
    assert (r[:, 6] >= 0).all() and (r[:, 7] & 0xFFFF < hkv).all()
    assert ((r[:, 7] >> 16) < n).all()

    say("timeline: capacity 3, then unregistered")
    buf.zero_()
    torch.cuda.synchronize()
    assert lib.ra_diag_timeline(ctypes.c_void_p(buf.data_ptr()), 3) == 0
    out2, lse2 = _run(lib, qd, kd, vd, c, rank)
    assert lib.ra_diag_timeline(None, 0) == 0
    rec = buf.cpu().numpy()
    assert np.count_nonzero(rec[:3, 0]) == 3 and not rec[3:].any()
    buf.zero_()
    torch.cuda.synchronize()
    out3, lse3 = _run(lib, qd, kd, vd, c, rank)
    assert not buf.cpu().numpy().any()
    for o, l_ in ((out2, lse2), (out3, lse3)):
        assert torch.equal(o, ref_out) and torch.equal(l_, ref_lse)
