"""Dense [prefix | fresh] mode (attn.dense: DenseAttentionManager, DensePlan).

Oracle pins (no library needed):
- attention over contiguous K/V equals torch's scaled_dot_product_attention
  (float64, explicit bottom-right causal / window mask, heads repeated for GQA);
- it equals the paged oracle on the same logical K/V (rows read back off the
  generator's page layout);
- the gather is checked on a hand-built pool whose every element names its
  (page, K|V, slot), so a wrong page, slot, half or row offset shows.

Library on the CPU: the dense planner's tiles are the prefill policy with a
row's keys starting at cu_k[r]; bad cu arrays and page tables are rejected; a
dense plan is refused by the paged entry points and vice versa.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _logical_kv(w, r):
    n = int(w.kv_len[r])
    ks, vs = [], []
    for j in range(n):
        page = int(w.kv_indices[w.kv_indptr[r] + j // w.page_size])
        ks.append(w.cache[page, 0, j % w.page_size])
        vs.append(w.cache[page, 1, j % w.page_size])
    return torch.stack(ks), torch.stack(vs)


def _dense_from_paged(w):
    """Contiguous bf16 K/V [sum kv_len, Hk, D] and cu_k of a paged case."""
    ks, vs = zip(*[_logical_kv(w, r) for r in range(w.batch)])
    cu_k = np.concatenate([[0], np.cumsum(w.kv_len)]).astype(np.int32)
    return torch.cat(ks), torch.cat(vs), cu_k


def _mask(n, L, causal, window_left):
    m = np.zeros((L, n), dtype=bool)
    for t in range(L):
        p = n - L + t
        for j in range(n):
            ok = (j <= p) if causal else True
            m[t, j] = ok and not (window_left >= 0 and j < p - window_left)
    return m


CASES = [
    dict(seed=71, page_size=4, head_dim=8, causal=True, window_left=-1),
    dict(seed=72, page_size=1, head_dim=16, causal=True, window_left=4),
    dict(seed=73, page_size=16, head_dim=8, causal=False, window_left=-1),
    dict(seed=74, page_size=2, head_dim=8, causal=False, window_left=6),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_dense_oracle_matches_sdpa(case):
    w = synth.random_case(case["seed"], page_size=case["page_size"], head_dim=case["head_dim"],
                          causal=case["causal"], window_left=case["window_left"], max_kv=30)
    k, v, cu_k = _dense_from_paged(w)
    out, lse = oracle.attention_dense(w.q, k, v, w.qo_indptr, cu_k, num_qo_heads=w.num_qo_heads,
                                      num_kv_heads=w.num_kv_heads, causal=w.causal,
                                      window_left=w.window_left)
    g = w.num_qo_heads // w.num_kv_heads
    for r in range(w.batch):
        L, n = int(w.q_len[r]), int(w.kv_len[r])
        if L == 0:
            continue
        K = k[cu_k[r]:cu_k[r + 1]].double().repeat_interleave(g, dim=1)
        V = v[cu_k[r]:cu_k[r + 1]].double().repeat_interleave(g, dim=1)
        q = w.q[w.qo_indptr[r]:w.qo_indptr[r + 1]].double()
        mask = torch.from_numpy(_mask(n, L, w.causal, w.window_left))
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(0, 1), K.transpose(0, 1).contiguous(), V.transpose(0, 1).contiguous(),
            attn_mask=mask)
        got = out[w.qo_indptr[r]:w.qo_indptr[r + 1]]
        assert np.max(np.abs(ref.transpose(0, 1).numpy() - got)) <= 1e-12
        logits = np.einsum("thd,jhd->thj", q.numpy(), K.numpy()) / math.sqrt(w.head_dim)
        logits = np.where(mask.numpy()[:, None, :], logits, -np.inf)
        m = logits.max(-1, keepdims=True)
        lref = (np.log(np.exp(logits - m).sum(-1, keepdims=True)) + m)[..., 0]
        assert np.max(np.abs(lref - lse[w.qo_indptr[r]:w.qo_indptr[r + 1]])) <= 1e-12


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_dense_oracle_equals_paged_oracle(case):
    w = synth.random_case(case["seed"], page_size=case["page_size"], head_dim=case["head_dim"],
                          causal=case["causal"], window_left=case["window_left"], max_kv=30)
    k, v, cu_k = _dense_from_paged(w)
    o1, l1 = oracle.attention_dense(w.q, k, v, w.qo_indptr, cu_k, num_qo_heads=w.num_qo_heads,
                                    num_kv_heads=w.num_kv_heads, causal=w.causal,
                                    window_left=w.window_left)
    o2, l2 = oracle.attention(w.q, w.cache, w.page_size, w.kv_indptr, w.kv_indices,
                              w.last_page_len, num_qo_heads=w.num_qo_heads,
                              num_kv_heads=w.num_kv_heads, qo_indptr=w.qo_indptr,
                              causal=w.causal, window_left=w.window_left)
    assert np.max(np.abs(o1 - o2), initial=0) <= 1e-12
    assert np.max(np.abs(l1 - l2), initial=0) <= 1e-12


def _labelled_pool(max_pages, ps, hk, d):
    """uint16 pool whose element (page, kv, slot, h, e) holds a value naming
    its page, half and slot (h and e ignored)."""
    pool = np.zeros((max_pages, 2, ps, hk, d), np.uint16)
    for p in range(max_pages):
        for kv in range(2):
            for s in range(ps):
                pool[p, kv, s] = 1 + p * 64 + kv * 32 + s
    return pool


def test_dense_gather_hand_case():
    ps, hk, d = 4, 1, 2
    pool = _labelled_pool(6, ps, hk, d)
    # row 0: prefix 5 tokens on pages [3, 1], 2 fresh; row 1: prefix 0, 1 fresh;
    # row 2: prefix 4 on page [5], 3 fresh
    cu_q = [0, 2, 3, 6]
    cu_k = [0, 7, 8, 15]
    indptr, idx = [0, 2, 2, 3], [3, 1, 5]
    kf = (1000 + np.arange(6)[:, None, None] * np.ones((1, hk, d))).astype(np.uint16)
    vf = kf + 500
    ko, vo = oracle.dense_gather(pool, ps, indptr, idx, cu_q, cu_k, kf, vf)
    want_k = [1 + 3 * 64 + s for s in range(4)] + [1 + 1 * 64 + 0] + [1000, 1001] + [1002] + \
             [1 + 5 * 64 + s for s in range(4)] + [1003, 1004, 1005]
    assert list(ko[:, 0, 0]) == want_k
    assert list(vo[:, 0, 0]) == [x + 32 if x < 1000 else x + 500 for x in want_k]
    # fresh-only refresh keeps the prefix rows it is given
    base = np.full_like(ko, 7)
    ko2, _ = oracle.dense_gather(pool, ps, indptr, idx, cu_q, cu_k, kf, vf, with_prefix=False,
                                 k_out=base, v_out=base)
    assert list(ko2[:, 0, 0]) == [7] * 5 + [1000, 1001, 1002] + [7] * 4 + [1003, 1004, 1005]


# ---- the library's host side ----

def _lib():
    return pytest.importorskip("paged_kv_attention_plan_amd.pkv",
                               reason="libpkv.so not built (python -m paged_kv_attention_plan_amd.build)")


def _dense_params(pkv, hq=8, hk=2, d=128, ps=16, causal=True, wl=-1, max_pages=1000):
    return pkv.plan_params("dense", num_qo_heads=hq, num_kv_heads=hk, head_dim=d, page_size=ps,
                           max_pages=max_pages, causal=causal, window_left=wl, num_cus=8)


@pytest.mark.parametrize("hq,hk,causal,wl", [(8, 2, True, -1), (4, 4, False, -1), (16, 2, True, 9),
                                             (32, 8, False, 40)])
def test_dense_plan_tiles_follow_prefill_policy(hq, hk, causal, wl):
    pkv = _lib()
    rng = np.random.default_rng(hq + hk + wl)
    B = 9
    L = rng.integers(0, 300, size=B)
    P = rng.integers(0, 500, size=B)
    L[2] = 0
    cu_q = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(L + P)]).astype(np.int32)
    plan = pkv.dense_plan_create(_dense_params(pkv, hq, hk, causal=causal, wl=wl), cu_q, cu_k)
    lay = [oracle.RowLayout(pages=None, kv_len=int(L[r] + P[r]), q_len=int(L[r])) for r in range(B)]
    rows = [r for r in range(B) if L[r] >= 1]
    want = oracle.prefill_policy(lay, rows, num_qo_heads=hq, num_kv_heads=hk, causal=causal,
                                 window_left=wl, qo_indptr=cu_q, kv_indptr=cu_k)
    got = [tuple(int(x) for x in t)[:10] for t in plan.prefill_tiles()]
    assert got == want
    oracle.check_prefill_cover(got, lay, rows, num_kv_heads=hk, causal=causal, window_left=wl)
    info = plan.info()
    assert info["total_q"] == cu_q[-1] and info["total_k"] == cu_k[-1]
    assert len(plan.decode_tiles()) == 0 and len(plan.write_slots()) == 0


@pytest.mark.parametrize("bad", ["q_gt_k", "cu_start", "decreasing", "few_pages", "page_oob",
                                 "half_table", "paged_api"])
def test_dense_plan_errors(bad):
    pkv = _lib()
    cu_q, cu_k = np.array([0, 3, 5]), np.array([0, 10, 14])
    ind, idx = np.array([0, 1, 2]), np.array([4, 7])  # ps 16: row 0 prefix 7, row 1 prefix 2
    p = _dense_params(pkv)
    if bad == "q_gt_k":
        cu_q = np.array([0, 11, 13])
    if bad == "cu_start":
        cu_k = np.array([1, 10, 14])
    if bad == "decreasing":
        cu_k = np.array([0, 10, 9])
    if bad == "few_pages":
        ind = np.array([0, 1, 1])
    if bad == "page_oob":
        idx = np.array([4, 5000])
    if bad == "half_table":
        idx = None
    if bad == "paged_api":
        with pytest.raises(pkv.PkvError, match="pkv_dense_plan_create"):
            pkv.plan_create(p, cu_q, ind, idx, np.array([1, 1]))
        return
    with pytest.raises(pkv.PkvError):
        pkv.dense_plan_create(p, cu_q, cu_k, ind, idx)


def test_dense_plan_refused_by_paged_calls_and_vice_versa():
    pkv = _lib()
    plan = pkv.dense_plan_create(_dense_params(pkv), [0, 2], [0, 5])
    v = ctypes.c_void_p(4096)
    null = ctypes.c_void_p(0)
    assert pkv._lib.pkv_run(plan.handle, v, v, v, None, v, plan.ws_bytes, null) == pkv.E_INVALID
    assert pkv._lib.pkv_append_kv(plan.handle, v, v, v, v, plan.ws_bytes, null) == pkv.E_INVALID
    assert pkv._lib.pkv_run_append(plan.handle, v, v, v, v, v, None, v, plan.ws_bytes,
                                   null) == pkv.E_INVALID
    with pytest.raises(pkv.PkvError, match="pkv_dense_plan_update"):
        pkv.plan_update(plan, [0, 2], [0, 1], [0], [2])
    w = synth.random_case(75, kind="prefill", page_size=4, head_dim=64, max_kv=20)
    paged = pkv.plan_create(pkv.plan_params("prefill", num_qo_heads=w.num_qo_heads,
                                            num_kv_heads=w.num_kv_heads, head_dim=64, page_size=4,
                                            max_pages=w.max_pages, num_cus=8),
                            w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len)
    assert pkv._lib.pkv_dense_run(paged.handle, v, v, v, v, None, v, paged.ws_bytes,
                                  null) == pkv.E_INVALID
    assert pkv._lib.pkv_dense_gather(paged.handle, v, v, v, v, v, 1, v, paged.ws_bytes,
                                     null) == pkv.E_INVALID
    # not uploaded yet
    assert pkv._lib.pkv_dense_run(plan.handle, v, v, v, v, None, v, plan.ws_bytes,
                                  null) == pkv.E_STATE


def test_dense_plan_update_replans():
    pkv = _lib()
    plan = pkv.dense_plan_create(_dense_params(pkv), [0, 2], [0, 5])
    n = pkv.dense_plan_update(plan, [0, 1, 40], [0, 3, 100])
    assert plan.info()["batch"] == 2 and plan.info()["total_k"] == 100 and n == plan.ws_bytes
