"""Context-only views (kv.plan, context_only_views): the page table of a step's
rows without the tokens the step appends.

Oracle pins (no library needed):
- a hand-worked case, including a row whose kept length ends exactly on a
  page boundary;
- to_compute = 0 leaves the page table unchanged;
- attention over the new views (every query sees every kept key) equals
  torch's scaled_dot_product_attention on the row's first kv_len - to_compute
  keys read straight off the generator's layout;
- invalid rows are rejected.

Library parity (CPU): pkv_context_only_views agrees with the oracle bit for
bit and rejects the same rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_hand_worked_views():
    # page_size 4.  row 0: pages [5, 2, 7], 11 tokens; drop 4 -> 7 tokens on [5, 2], lpl 3.
    # row 1: page [1], 4 tokens; drop 3 -> 1 token, lpl 1.
    # row 2: pages [0, 3], 5 tokens; drop 1 -> 4 tokens: page 3 goes, page 0 is full (lpl 4).
    ptr, idx, lpl, qo = oracle.context_only_views(
        4, [0, 3, 4, 6], [5, 2, 7, 1, 0, 3], [3, 4, 1], to_compute=[4, 3, 1], query_spans=[2, 1, 3])
    assert list(ptr) == [0, 2, 3, 4]
    assert list(idx) == [5, 2, 1, 0]
    assert list(lpl) == [3, 1, 4]
    assert list(qo) == [0, 2, 3, 6]


def test_nothing_appended_keeps_the_table():
    w = synth.random_case(31, batch=5, page_size=4, max_kv=40)
    spans = np.array([3, 0, 1, 2, 5])
    ptr, idx, lpl, qo = oracle.context_only_views(w.page_size, w.kv_indptr, w.kv_indices,
                                                  w.last_page_len, np.zeros(5, np.int64), spans)
    assert np.array_equal(ptr, w.kv_indptr) and np.array_equal(idx, w.kv_indices)
    assert np.array_equal(lpl, w.last_page_len)
    assert list(qo) == [0, 3, 3, 4, 6, 11]


def _logical_kv(w, r, n):
    """The first n tokens of row r read back the way the generator laid them
    out (token j on page kv_indices[kv_indptr[r] + j // ps], slot j % ps)."""
    ks, vs = [], []
    for j in range(n):
        page = int(w.kv_indices[w.kv_indptr[r] + j // w.page_size])
        ks.append(w.cache[page, 0, j % w.page_size].double().numpy())
        vs.append(w.cache[page, 1, j % w.page_size].double().numpy())
    return np.stack(ks), np.stack(vs)


@pytest.mark.parametrize("seed,page_size", [(41, 1), (42, 4), (43, 16), (44, 2)])
def test_attention_over_views_matches_sdpa_on_kept_keys(seed, page_size):
    w = synth.random_case(seed, batch=4, page_size=page_size, max_kv=36, head_dim=8)
    rng = np.random.default_rng(seed)
    tc = np.array([rng.integers(0, int(n)) for n in w.kv_len])
    spans = np.array([rng.integers(1, int(n) - int(t) + 1) for n, t in zip(w.kv_len, tc)])
    ptr, idx, lpl, qo = oracle.context_only_views(page_size, w.kv_indptr, w.kv_indices,
                                                  w.last_page_len, tc, spans)
    q = torch.randn(int(qo[-1]), w.num_qo_heads, w.head_dim, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    out, lse = oracle.attention(q, w.cache, page_size, ptr, idx, lpl, num_qo_heads=w.num_qo_heads,
                                num_kv_heads=w.num_kv_heads, qo_indptr=qo, causal=False,
                                window_left=-1)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        kept = int(w.kv_len[r] - tc[r])
        K, V = _logical_kv(w, r, kept)
        Kt = torch.from_numpy(K).repeat_interleave(g, dim=1)
        Vt = torch.from_numpy(V).repeat_interleave(g, dim=1)
        qr = q[qo[r]:qo[r + 1]].double()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr.transpose(0, 1), Kt.transpose(0, 1).contiguous(), Vt.transpose(0, 1).contiguous())
        assert np.max(np.abs(ref.transpose(0, 1).numpy() - out[qo[r]:qo[r + 1]])) <= 1e-12
        logits = np.einsum("thd,jhd->thj", qr.numpy(), Kt.numpy()) / math.sqrt(w.head_dim)
        lref = np.log(np.exp(logits - logits.max(-1, keepdims=True)).sum(-1)) + logits.max(-1)
        assert np.max(np.abs(lref - lse[qo[r]:qo[r + 1]])) <= 1e-12


@pytest.mark.parametrize("tc,spans", [([4, 0], [1, 1]), ([-1, 0], [1, 1]), ([0, 0], [1, -1])])
def test_invalid_rows_are_rejected(tc, spans):
    # row 0 holds 4 tokens (one full page of 4), row 1 holds 2
    with pytest.raises(oracle.OracleError):
        oracle.context_only_views(4, [0, 1, 2], [0, 1], [4, 2], tc, spans)


# ---- the library's host function ----

def _lib():
    return pytest.importorskip("paged_kv_attention_plan_amd.pkv",
                               reason="libpkv.so not built (python -m paged_kv_attention_plan_amd.build)")


@pytest.mark.parametrize("seed,page_size", [(51, 1), (52, 4), (53, 16), (54, 32), (55, 8)])
def test_library_matches_oracle(seed, page_size):
    pkv = _lib()
    w = synth.random_case(seed, batch=7, page_size=page_size, max_kv=90)
    rng = np.random.default_rng(seed)
    tc = np.array([rng.integers(0, int(n)) for n in w.kv_len])
    spans = rng.integers(0, 9, size=w.batch)
    want = oracle.context_only_views(page_size, w.kv_indptr, w.kv_indices, w.last_page_len, tc, spans)
    got = pkv.context_only_views(page_size, w.kv_indptr, w.kv_indices, w.last_page_len, tc, spans)
    for a, b in zip(want, got):
        assert a.dtype == b.dtype and np.array_equal(a, b)


@pytest.mark.parametrize("tc,spans", [([4, 0], [1, 1]), ([-1, 0], [1, 1]), ([0, 0], [1, -1])])
def test_library_rejects_invalid_rows(tc, spans):
    pkv = _lib()
    with pytest.raises(pkv.PkvError, match="to_compute|query_spans"):
        pkv.context_only_views(4, [0, 1, 2], [0, 1], [4, 2], tc, spans)


def test_library_rejects_malformed_table():
    pkv = _lib()
    with pytest.raises(pkv.PkvError):
        pkv.context_only_views(4, [0, 1, 2], [0, 1], [5, 2], [0, 0], [1, 1])  # lpl > page_size
    with pytest.raises(pkv.PkvError):
        pkv.context_only_views(3, [0, 1], [0], [2], [0], [1])  # page_size not a power of two
