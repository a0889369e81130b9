"""The stored tiny-decode fixture still matches the oracle, and the planner
cover checkers accept valid plans and reject broken ones."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_decode.json")


def test_tiny_decode_golden_matches_oracle():
    doc = json.load(open(GOLDEN))
    w = synth.make_workload("tiny_decode")
    assert [int(x) for x in w.kv_len] == doc["kv_len"]
    assert [int(x) for x in w.kv_indices] == doc["kv_indices"]
    out, lse = oracle.attention(w.q, w.cache, w.page_size, w.kv_indptr, w.kv_indices,
                                w.last_page_len, num_qo_heads=4, num_kv_heads=2)
    assert np.max(np.abs(out - np.array(doc["out"]))) < 1e-13
    assert np.max(np.abs(lse - np.array(doc["lse"]))) < 1e-13
    slots = oracle.write_slots(16, w.kv_indptr, w.kv_indices, w.last_page_len)
    assert list(slots) == doc["write_slots"]


def _layout(w):
    return oracle.decode_csr(w.page_size, w.kv_indptr, w.kv_indices, w.last_page_len,
                             max_pages=w.max_pages, qo_indptr=w.qo_indptr)


@pytest.mark.parametrize("window_left", [-1, 0, 9, 40])
def test_decode_policy_passes_cover_check(window_left):
    w = synth.random_case(30, kind="decode", batch=6, page_size=4, max_kv=120,
                          window_left=window_left)
    lay = _layout(w)
    rows = list(range(w.batch))
    tiles, merges, cap, n_slots, work = oracle.decode_policy(
        lay, rows, page_size=4, num_kv_heads=2, window_left=window_left, num_cus=2,
        qo_indptr=w.qo_indptr, kv_indptr=w.kv_indptr, group=w.num_qo_heads // 2,
        waves_per_cu=8, min_chunk_pages=2)
    oracle.check_decode_cover(tiles, merges, lay, rows, num_kv_heads=2, window_left=window_left,
                              n_slots=n_slots)
    if window_left in (-1, 40):
        assert any(t[6] >= 0 for t in tiles), "the case should exercise split-KV"
        # a broken plan: shift one chunk boundary
        bad = list(tiles)
        i = next(k for k, t in enumerate(bad) if t[6] >= 0)
        t = bad[i]
        bad[i] = (t[0], t[1], t[2] + 1, t[3], t[4], t[5], t[6], t[7])
        with pytest.raises(AssertionError):
            oracle.check_decode_cover(bad, merges, lay, rows, num_kv_heads=2,
                                      window_left=window_left, n_slots=n_slots)
    with pytest.raises(AssertionError):
        oracle.check_decode_cover(tiles[1:], merges, lay, rows, num_kv_heads=2,
                                  window_left=window_left, n_slots=n_slots)


@pytest.mark.parametrize("causal,window_left", [(True, -1), (True, 5), (False, -1), (False, 3)])
def test_prefill_policy_passes_cover_check(causal, window_left):
    w = synth.random_case(31, kind="prefill", batch=5, num_qo_heads=8, num_kv_heads=1,
                          page_size=4, max_kv=60, causal=causal, window_left=window_left)
    lay = _layout(w)
    rows = [r for r in range(w.batch) if lay[r].q_len > 0]
    tiles = oracle.prefill_policy(lay, rows, num_qo_heads=8, num_kv_heads=1, causal=causal,
                                  window_left=window_left, qo_indptr=w.qo_indptr,
                                  kv_indptr=w.kv_indptr)
    oracle.check_prefill_cover(tiles, lay, rows, num_kv_heads=1, causal=causal,
                               window_left=window_left)
    t = tiles[0]
    bad = [(t[0], t[1], t[2], t[3], t[4] + 1, t[5], *t[6:])] + tiles[1:]
    if t[4] + 1 > 0:
        with pytest.raises(AssertionError):
            oracle.check_prefill_cover(bad, lay, rows, num_kv_heads=1, causal=causal,
                                       window_left=window_left)
