"""The pins are sharp: plant a plausible mistake in the oracle (on the CPU) and check
that at least one pin fails. Each mutation is undone by monkeypatch afterwards."""

import numpy as np
import pytest

from oracle import attention as A
from tests import test_oracle_pins as pins


def _expect_pin_failure(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(A, "score_scale", lambda d: 1.0)
    _expect_pin_failure(pins.test_t5_torch_sdpa_fp64, 1, 1)
    _expect_pin_failure(pins.test_t1_bruteforce_50_digits, False, False, 1, 1, 3, 12)


def test_strict_causal_mask_is_caught(monkeypatch):
    monkeypatch.setattr(A, "causal_allowed", lambda pq, pk: pk[None, :] < pq[:, None])
    _expect_pin_failure(pins.test_t1_bruteforce_50_digits, True, False, 2, 1, 4, 16)
    _expect_pin_failure(pins.test_t6_closed_forms, True)


def test_wrong_zigzag_partner_chunk_is_caught(monkeypatch):
    orig = A.chunk_positions

    def bad(owner, rows, c, zigzag):
        p = orig(owner, rows, c, zigzag)
        if zigzag:
            m = rows // 2
            p = p.copy()
            p[m:] -= m   # partner chunk 2c-2-i instead of 2c-1-i
        return p
    monkeypatch.setattr(A, "chunk_positions", bad)
    _expect_pin_failure(pins.test_t4_share_rows_equal_full_sequence_rows, True)


def test_wrong_gqa_map_is_caught(monkeypatch):
    monkeypatch.setattr(A, "kv_head", lambda h, hq, hkv: h % hkv)
    _expect_pin_failure(pins.test_t5_torch_sdpa_fp64, 4, 2)


def test_swapped_merge_weights_are_caught(monkeypatch):
    orig = A.merge
    monkeypatch.setattr(A, "merge", lambda oa, la, ob, lb: orig(oa, lb, ob, la))
    import oracle
    monkeypatch.setattr(oracle, "merge", A.merge)
    _expect_pin_failure(pins.test_t7_partials_merge_to_fused, False, False)


def test_reversed_ring_direction_is_caught(monkeypatch):
    monkeypatch.setattr(A, "ring_blocks",
                        lambda c, rank, b=0, e=None: [(rank + t) % c for t in range(b, c if e is None else e)])
    _expect_pin_failure(pins.test_ring_direction_rank_i_sends_to_i_plus_1)


def test_unpinned_mutation_control():
    # sanity: the unmutated pins pass when called directly
    pins.test_t5_torch_sdpa_fp64(4, 2)
    pins.test_t4_share_rows_equal_full_sequence_rows(True)
    assert np.isfinite(A.score_scale(64))


def test_document_start_off_by_one_is_caught(monkeypatch):
    def bad(pq, pk, ds):
        lo = np.asarray(ds, dtype=np.int64)[pq]
        return (pk[None, :] <= pq[:, None]) & (pk[None, :] > lo[:, None])   # drops the first token
    monkeypatch.setattr(A, "document_allowed", bad)
    _expect_pin_failure(pins.test_t8_documents_equal_separate_causal_attention, [10, 1, 1, 20, 32])


def test_document_mask_ignored_is_caught(monkeypatch):
    monkeypatch.setattr(A, "document_allowed", lambda pq, pk, ds: A.causal_allowed(pq, pk))
    _expect_pin_failure(pins.test_t8_documents_equal_separate_causal_attention, [17, 15, 16, 16])
    _expect_pin_failure(pins.test_t8_documents_bruteforce_50_digits, True)
