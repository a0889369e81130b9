"""Pins for the CPU oracle: each test checks it against something other than
itself -- a scalar brute force, closed forms, torch's SDPA on contiguous K/V,
invariants of the page table, and a hand-worked example.  The mutation tests
plant plausible mistakes in the oracle and check that some pin catches each.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import reference as oa
import synth


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _run(w, **kw):
    return oracle.attention(w.q, w.cache, w.page_size, w.kv_indptr, w.kv_indices, w.last_page_len,
                            num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                            qo_indptr=w.qo_indptr, causal=w.causal, window_left=w.window_left, **kw)


def _logical_kv(w, r):
    """Row r's K/V read back the way the generator laid them out: token j on
    page kv_indices[kv_indptr[r] + j // ps] at slot j % ps (independent of the
    oracle's gather)."""
    n = int(w.kv_len[r])
    ks, vs = [], []
    for j in range(n):
        page = int(w.kv_indices[w.kv_indptr[r] + j // w.page_size])
        ks.append(w.cache[page, 0, j % w.page_size].float().double().numpy())
        vs.append(w.cache[page, 1, j % w.page_size].float().double().numpy())
    return np.stack(ks), np.stack(vs)


def _mask(n, L, causal, window_left):
    """Boolean [L, n]: query t (at position n - L + t) may see key j."""
    m = np.zeros((L, n), dtype=bool)
    for t in range(L):
        p = n - L + t
        for j in range(n):
            ok = (j <= p) if causal else True
            if window_left >= 0 and j < p - window_left:
                ok = False
            m[t, j] = ok
    return m


CASES = [
    dict(seed=1, page_size=1, head_dim=8, causal=True, window_left=-1),
    dict(seed=2, page_size=2, head_dim=8, causal=True, window_left=3),
    dict(seed=3, page_size=4, head_dim=4, causal=False, window_left=-1),
    dict(seed=4, page_size=16, head_dim=8, causal=True, window_left=0),
    dict(seed=5, page_size=4, head_dim=8, causal=False, window_left=5),
    dict(seed=6, page_size=16, head_dim=64, causal=True, window_left=-1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_bruteforce_matches_vectorized(case):
    w = synth.random_case(case["seed"], page_size=case["page_size"], head_dim=case["head_dim"],
                          causal=case["causal"], window_left=case["window_left"], max_kv=30)
    o1, l1 = _run(w)
    o2, l2 = oracle.attention_bruteforce(w.q, w.cache, w.page_size, w.kv_indptr, w.kv_indices,
                                         w.last_page_len, num_qo_heads=w.num_qo_heads,
                                         num_kv_heads=w.num_kv_heads, qo_indptr=w.qo_indptr,
                                         causal=w.causal, window_left=w.window_left)
    assert np.max(np.abs(o1 - o2), initial=0) <= 1e-12
    assert np.max(np.abs(l1 - l2), initial=0) <= 1e-12


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_matches_sdpa_on_contiguous_kv(case):
    """torch's scaled_dot_product_attention (float64, explicit mask, heads
    repeated for GQA) on the row's K/V read straight off the generator's layout;
    lse against scipy's logsumexp."""
    w = synth.random_case(case["seed"], page_size=case["page_size"], head_dim=case["head_dim"],
                          causal=case["causal"], window_left=case["window_left"], max_kv=30)
    out, lse = _run(w)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        L, n = int(w.q_len[r]), int(w.kv_len[r])
        if L == 0:
            continue
        K, V = _logical_kv(w, r)                      # [n, Hk, D]
        q = w.q[w.qo_indptr[r]:w.qo_indptr[r + 1]].double()          # [L, Hq, D]
        Kt = torch.from_numpy(K).repeat_interleave(g, dim=1)           # [n, Hq, D]
        Vt = torch.from_numpy(V).repeat_interleave(g, dim=1)
        mask = torch.from_numpy(_mask(n, L, w.causal, w.window_left))
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(0, 1), Kt.transpose(0, 1), Vt.transpose(0, 1), attn_mask=mask)
        got = out[w.qo_indptr[r]:w.qo_indptr[r + 1]]
        assert np.max(np.abs(ref.transpose(0, 1).numpy() - got)) <= 1e-12
        logits = np.einsum("thd,jhd->thj", q.numpy(), Kt.numpy()) / math.sqrt(q.shape[-1])
        logits = np.where(mask.numpy()[:, None, :], logits, -np.inf)
        assert np.max(np.abs(logsumexp(logits, axis=-1) - lse[w.qo_indptr[r]:w.qo_indptr[r + 1]])) <= 1e-12


@pytest.mark.parametrize("window_left", [-1, 0, 2, 7])
@pytest.mark.parametrize("causal", [True, False])
def test_zero_query_closed_form(causal, window_left):
    """q = 0 makes every visible logit 0: out is the mean of the visible V rows
    and lse = ln(number of visible keys).  Pins causal alignment to the end of
    the KV, the window bound and the page gather."""
    w = synth.random_case(11, page_size=4, head_dim=8, causal=causal, window_left=window_left,
                          max_kv=25, batch=4)
    w.q.zero_()
    out, lse = _run(w)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        L, n = int(w.q_len[r]), int(w.kv_len[r])
        _, V = _logical_kv(w, r)
        for t in range(L):
            p = n - L + t
            hi = p if causal else n - 1
            lo = 0 if window_left < 0 else max(0, p - window_left)
            for h in range(w.num_qo_heads):
                exp_o = V[lo:hi + 1, h // g].mean(axis=0)
                assert np.allclose(out[w.qo_indptr[r] + t, h], exp_o, atol=1e-13, rtol=0)
                assert abs(lse[w.qo_indptr[r] + t, h] - math.log(hi - lo + 1)) <= 1e-13


def test_single_visible_key_returns_that_value():
    """window_left = 0 under causal masking leaves only the query's own key:
    out = v[p] exactly and lse = its scaled logit."""
    w = synth.random_case(12, page_size=4, head_dim=8, causal=True, window_left=0, max_kv=20)
    out, lse = _run(w)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        L, n = int(w.q_len[r]), int(w.kv_len[r])
        K, V = _logical_kv(w, r)
        for t in range(L):
            p = n - L + t
            for h in range(w.num_qo_heads):
                assert np.array_equal(out[w.qo_indptr[r] + t, h], V[p, h // g])
                qv = w.q[w.qo_indptr[r] + t, h].double().numpy()
                assert abs(lse[w.qo_indptr[r] + t, h] - qv @ K[p, h // g] / math.sqrt(8)) <= 1e-12


def test_hand_worked_example():
    """head_dim 4, scale 1/2.  q = (2,0,0,0) and keys k_j = (j,0,0,0) give
    logits 0, 1, 2; values v_j = (j, 1, -j, 0).  By hand:
        lse = ln(1 + e + e^2),  out = ((e + 2e^2)/Z, 1, -(e + 2e^2)/Z, 0)."""
    cache = torch.zeros(3, 2, 2, 1, 4, dtype=torch.bfloat16)
    # three keys on pages 2 then 0 (page size 2): positions 0,1 on page 2; 2 on page 0
    pos_to = {0: (2, 0), 1: (2, 1), 2: (0, 0)}
    for j, (pg, s) in pos_to.items():
        cache[pg, 0, s, 0] = torch.tensor([j, 0, 0, 0], dtype=torch.bfloat16)
        cache[pg, 1, s, 0] = torch.tensor([j, 1, -j, 0], dtype=torch.bfloat16)
    q = torch.tensor([[[2.0, 0, 0, 0]]], dtype=torch.bfloat16)
    out, lse = oracle.attention(q, cache, 2, np.array([0, 2]), np.array([2, 0]), np.array([1]),
                                num_qo_heads=1, num_kv_heads=1)
    e = math.e
    Z = 1 + e + e * e
    a = (e + 2 * e * e) / Z
    assert abs(lse[0, 0] - math.log(Z)) < 1e-14
    assert np.allclose(out[0, 0], [a, 1.0, -a, 0.0], atol=1e-14, rtol=0)


def test_page_relabelling_is_exact():
    """Moving pages to other physical ids (data moved with them) changes nothing."""
    w = synth.random_case(13, page_size=4, head_dim=8, max_kv=30, extra_pages=7)
    o1, l1 = _run(w)
    rng = np.random.default_rng(0)
    perm = rng.permutation(w.max_pages)
    cache2 = torch.empty_like(w.cache)
    cache2[torch.from_numpy(perm)] = w.cache
    w2 = synth.Workload(**{**w.__dict__, "cache": cache2, "kv_indices": perm[w.kv_indices].astype(np.int32)})
    o2, l2 = _run(w2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_size_invariance():
    """The same logical K/V laid out with page sizes 1, 4, 16 and one page
    larger than every row give the same attention (to rounding)."""
    base = synth.random_case(14, page_size=1, head_dim=8, max_kv=30, extra_pages=0)
    ref_o, ref_l = _run(base)
    for ps in (4, 16, 64):
        Kall = [_logical_kv(base, r) for r in range(base.batch)]
        n_pages = [(int(n) + ps - 1) // ps for n in base.kv_len]
        cache = torch.zeros(sum(n_pages), 2, ps, base.num_kv_heads, base.head_dim, dtype=torch.bfloat16)
        indices = np.arange(sum(n_pages))[::-1].copy().astype(np.int32)  # reversed physical order
        indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
        for r, (K, V) in enumerate(Kall):
            for j in range(len(K)):
                pg = indices[indptr[r] + j // ps]
                cache[pg, 0, j % ps] = torch.from_numpy(K[j]).to(torch.bfloat16)
                cache[pg, 1, j % ps] = torch.from_numpy(V[j]).to(torch.bfloat16)
        lpl = (((base.kv_len - 1) % ps) + 1).astype(np.int32)
        o, l = oracle.attention(base.q, cache, ps, indptr, indices, lpl,
                                num_qo_heads=base.num_qo_heads, num_kv_heads=base.num_kv_heads,
                                qo_indptr=base.qo_indptr, causal=True, window_left=-1)
        assert np.max(np.abs(o - ref_o)) <= 1e-12 and np.max(np.abs(l - ref_l)) <= 1e-12


def test_merge_partials_against_sdpa():
    """Attention over disjoint key chunks (each by SDPA), merged by
    merge_partials, equals attention over all keys (by SDPA)."""
    rng = np.random.default_rng(3)
    n, D = 37, 16
    q = torch.from_numpy(rng.standard_normal((2, 1, D)))
    K = torch.from_numpy(rng.standard_normal((2, n, D)))
    V = torch.from_numpy(rng.standard_normal((2, n, D)))
    full = torch.nn.functional.scaled_dot_product_attention(q, K, V)[:, 0].numpy()
    full_lse = logsumexp((q @ K.transpose(1, 2)).numpy()[:, 0] / math.sqrt(D), axis=-1)
    cuts = [0, 5, 6, 20, n]
    parts_o, parts_l = [], []
    for a, b in zip(cuts, cuts[1:]):
        parts_o.append(torch.nn.functional.scaled_dot_product_attention(q, K[:, a:b], V[:, a:b])[:, 0].numpy())
        parts_l.append(logsumexp((q @ K[:, a:b].transpose(1, 2)).numpy()[:, 0] / math.sqrt(D), axis=-1))
    o, l = oracle.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.max(np.abs(o - full)) <= 1e-12 and np.max(np.abs(l - full_lse)) <= 1e-12


def test_decode_equals_prefill_with_one_token():
    w = synth.random_case(15, kind="decode", page_size=4, head_dim=8, max_kv=30)
    o1, l1 = oracle.attention(w.q, w.cache, w.page_size, w.kv_indptr, w.kv_indices,
                              w.last_page_len, num_qo_heads=4, num_kv_heads=2)
    o2, l2 = _run(w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_stale_slots_do_not_matter():
    """NaN in unused pages and past the last token of each row changes nothing."""
    a = synth.random_case(16, page_size=8, head_dim=8, max_kv=30, stale="zero")
    b = synth.random_case(16, page_size=8, head_dim=8, max_kv=30, stale="nan")
    oa_, la_ = _run(a)
    ob_, lb_ = _run(b)
    assert np.array_equal(oa_, ob_) and np.array_equal(la_, lb_)


def test_write_slots_match_generator_layout():
    """Every query token's slot is where the generator put that position."""
    w = synth.random_case(17, page_size=4, head_dim=8, max_kv=30)
    slots = oracle.write_slots(w.page_size, w.kv_indptr, w.kv_indices, w.last_page_len,
                               qo_indptr=w.qo_indptr)
    k = 0
    for r in range(w.batch):
        n, L = int(w.kv_len[r]), int(w.q_len[r])
        for j in range(n - L, n):
            page = int(w.kv_indices[w.kv_indptr[r] + j // w.page_size])
            assert slots[k] == page * w.page_size + j % w.page_size
            k += 1
    assert k == len(slots)


def test_decode_write_slot_is_last_page_at_lpl_minus_one():
    w = synth.random_case(18, kind="decode", page_size=16, head_dim=8, max_kv=60)
    slots = oracle.write_slots(16, w.kv_indptr, w.kv_indices, w.last_page_len)
    for r in range(w.batch):
        last = int(w.kv_indices[w.kv_indptr[r + 1] - 1])
        assert slots[r] == last * 16 + int(w.last_page_len[r]) - 1


def test_apply_append_touches_only_slots():
    w = synth.random_case(19, kind="decode", page_size=4, head_dim=8, max_kv=30, new_tokens=True)
    slots = oracle.write_slots(4, w.kv_indptr, w.kv_indices, w.last_page_len)
    before = _bits(w.cache)
    after = oracle.apply_append(before, slots, _bits(w.k_new), _bits(w.v_new), 4)
    changed = np.argwhere((after != before).any(axis=(3, 4)))
    for t, s in enumerate(slots):
        assert np.array_equal(after[s // 4, 0, s % 4], _bits(w.k_new)[t])
        assert np.array_equal(after[s // 4, 1, s % 4], _bits(w.v_new)[t])
    allowed = {(int(s) // 4, kv, int(s) % 4) for s in slots for kv in (0, 1)}
    assert {tuple(c) for c in changed} <= allowed


def test_mixed_permutation_hand_case():
    # rows: q_len 1, 3, 0, 1, 2 -> decode rows 0, 3; prompt rows 1, 4
    qo = np.array([0, 1, 4, 4, 5, 7])
    dec, pre, perm = oracle.mixed_permutation(qo, max_prefill_rows=2)
    assert list(dec) == [0, 3] and list(pre) == [1, 4] and list(perm) == [1, 2, 3, 5, 6]
    with pytest.raises(oracle.OracleError):
        oracle.mixed_permutation(qo, max_prefill_rows=1)


@pytest.mark.parametrize("bad", ["lpl0", "lpl_big", "no_pages", "page_oob", "qlen"])
def test_csr_validation(bad):
    indptr, idx, lpl, qo = np.array([0, 2, 3]), np.array([0, 1, 2]), np.array([3, 4]), np.array([0, 2, 3])
    if bad == "lpl0":
        lpl = np.array([0, 4])
    if bad == "lpl_big":
        lpl = np.array([5, 4])
    if bad == "no_pages":
        indptr = np.array([0, 0, 3])
    if bad == "page_oob":
        idx = np.array([0, 1, 9])
    if bad == "qlen":
        qo = np.array([0, 2, 8])
    with pytest.raises(oracle.OracleError):
        oracle.decode_csr(4, indptr, idx, lpl, max_pages=4, qo_indptr=qo)


def test_csr_lengths_closed_form():
    lay = oracle.decode_csr(4, np.array([0, 2, 3]), np.array([0, 1, 2]), np.array([3, 4]), max_pages=4)
    assert [l.kv_len for l in lay] == [7, 4]


# ---- planted mistakes: every one must be caught by one of the pins above ----

def _pins_pass():
    """Run a compact set of the pins; True if all hold."""
    try:
        for c in CASES[:5]:
            test_matches_sdpa_on_contiguous_kv(c)
        for causal in (True, False):
            for wl in (-1, 2):
                test_zero_query_closed_form(causal, wl)
        test_hand_worked_example()
        test_single_visible_key_returns_that_value()
        return True
    except AssertionError:
        return False


def _mut_visible_off_by_one(p, n, causal, w):
    hi = p if causal else n - 1
    lo = 0 if w < 0 else max(0, p - w + 1)
    return lo, hi


def _mut_causal_exclusive(p, n, causal, w):
    hi = (p - 1 if p > 0 else 0) if causal else n - 1
    lo = 0 if w < 0 else max(0, p - w)
    return lo, hi


def _mut_position_top_left(n, L, t):
    return t


def _mut_kv_swapped(cache, pages, kv_len, page_size):
    K, V = _orig_gather(cache, pages, kv_len, page_size)
    return V, K


def _mut_page_order(cache, pages, kv_len, page_size):
    return _orig_gather(cache, pages[::-1], kv_len, page_size)


_orig_gather = oa.gather_row_kv


@pytest.mark.parametrize("name,target,repl", [
    ("window_off_by_one", "visible_keys", _mut_visible_off_by_one),
    ("causal_excludes_self", "visible_keys", _mut_causal_exclusive),
    ("causal_top_left", "query_position", _mut_position_top_left),
    ("k_v_swapped", "gather_row_kv", _mut_kv_swapped),
    ("pages_reversed", "gather_row_kv", _mut_page_order),
])
def test_planted_mistakes_are_caught(monkeypatch, name, target, repl):
    assert _pins_pass()
    monkeypatch.setattr(oa, target, repl)
    assert not _pins_pass(), f"planted mistake {name} went unnoticed"


def test_planted_wrong_scale_is_caught(monkeypatch):
    orig = oa._attend_head

    def wrong(qh, K, V, pos, kv_len, causal, window_left, scale):
        return orig(qh, K, V, pos, kv_len, causal, window_left, scale * 2)

    monkeypatch.setattr(oa, "_attend_head", wrong)
    assert not _pins_pass()


def test_planted_wrong_gqa_mapping_is_caught(monkeypatch):
    """Reading KV head h % Hk instead of h // group."""
    monkeypatch.setattr(oa, "kv_head_of", lambda h, hq, hk: h % hk)
    assert not _pins_pass()
