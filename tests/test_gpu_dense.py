"""Dense [prefix | fresh] mode on the GPU (attn.dense DenseAttentionManager).

- pkv_dense_gather builds the contiguous K/V bit for bit as the oracle does
  (prefix from the pages, fresh rows after it; and the fresh-only refresh);
- pkv_dense_run matches the dense oracle within the tolerances, over several
  query blocks and a ragged tail, for both head dims, GQA and MHA, causal and
  not, with and without a window;
- on the same logical K/V its output is bit-identical to pkv_run over the
  pages (the tiles differ only in where a key is read from);
- the full-size ragged-prefill shape in dense mode agrees with the paged run
  bit for bit and with the oracle on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, gpu_run, oracle_all, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _fresh_rows(w):
    """Indices (into the flat [pages * ps] token rows of each half) of every
    row's last q_len tokens, in q order: the step's fresh K/V as the pool
    holds them."""
    flat = []
    for r in range(w.batch):
        n, L = int(w.kv_len[r]), int(w.q_len[r])
        for j in range(n - L, n):
            page = int(w.kv_indices[w.kv_indptr[r] + j // w.page_size])
            flat.append(page * w.page_size + j % w.page_size)
    return torch.tensor(flat, dtype=torch.int64, device=w.q.device)


def _fresh_kv(w):
    idx = _fresh_rows(w)
    hk, d = w.num_kv_heads, w.head_dim
    k = w.cache[:, 0].reshape(-1, hk, d)[idx].contiguous()
    v = w.cache[:, 1].reshape(-1, hk, d)[idx].contiguous()
    return k, v


def _dense(pkv, w, with_pages=True):
    """Dense plan over w's rows (prefix = all but the last q_len tokens),
    uploaded, with the contiguous K/V gathered on the GPU."""
    cu_q = w.qo_indptr.astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(w.kv_len)]).astype(np.int32)
    params = pkv.plan_params("dense", num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                             head_dim=w.head_dim, page_size=w.page_size, max_pages=w.max_pages,
                             causal=w.causal, window_left=w.window_left)
    plan = pkv.dense_plan_create(params, cu_q, cu_k, w.kv_indptr if with_pages else None,
                                 w.kv_indices if with_pages else None)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=w.q.device)
    pkv.plan_upload(plan, ws)
    kf, vf = _fresh_kv(w)
    K = int(cu_k[-1])
    k = torch.full((K, w.num_kv_heads, w.head_dim), float("nan"), dtype=torch.bfloat16,
                   device=w.q.device)
    v = torch.full_like(k, float("nan"))
    pkv.dense_gather(plan, w.cache, kf, vf, k, v, ws, with_prefix=True)
    return plan, ws, k, v, kf, vf, cu_q, cu_k


@pytest.mark.parametrize("seed,ps", [(700, 16), (701, 4), (702, 1)])
def test_dense_gather_bit_exact(pkv, gpu, seed, ps):
    say(f"case dense gather seed={seed} ps={ps}")
    w = synth.random_case(seed, kind="prefill", batch=7, num_qo_heads=8, num_kv_heads=2,
                          head_dim=128, page_size=ps, max_kv=300, stale="nan", device=gpu)
    plan, ws, k, v, kf, vf, cu_q, cu_k = _dense(pkv, w)
    torch.cuda.synchronize()
    want_k, want_v = oracle.dense_gather(_bits(w.cache), ps, w.kv_indptr, w.kv_indices, cu_q, cu_k,
                                         _bits(kf), _bits(vf))
    assert np.array_equal(_bits(k), want_k) and np.array_equal(_bits(v), want_v)
    # fresh-only refresh over a buffer whose prefixes are already in place
    kf2 = torch.randn_like(kf, dtype=torch.float32).to(torch.bfloat16)
    vf2 = torch.randn_like(vf, dtype=torch.float32).to(torch.bfloat16)
    pkv.dense_gather(plan, None, kf2, vf2, k, v, ws, with_prefix=False)
    torch.cuda.synchronize()
    want_k2, want_v2 = oracle.dense_gather(None, ps, None, None, cu_q, cu_k, _bits(kf2), _bits(vf2),
                                           with_prefix=False, k_out=want_k, v_out=want_v)
    assert np.array_equal(_bits(k), want_k2) and np.array_equal(_bits(v), want_v2)


DENSE = [
    # (seed, head_dim, Hq, Hk, page_size, causal, window)
    (710, 128, 32, 8, 16, True, -1),
    (711, 64, 8, 8, 4, True, -1),
    (712, 128, 8, 1, 1, True, 7),
    (713, 64, 16, 2, 32, False, -1),
    (714, 128, 4, 2, 16, False, 40),
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: f"s{c[0]}-D{c[1]}-g{c[2]//c[3]}-ps{c[4]}-c{int(c[5])}-w{c[6]}")
def test_dense_run_matches_oracle_and_paged(pkv, gpu, case):
    seed, D, hq, hk, ps, causal, wl = case
    say(f"case dense run seed={seed} D={D} Hq={hq} Hk={hk} ps={ps} causal={causal} window={wl}")
    w = synth.random_case(seed, kind="prefill", batch=6, num_qo_heads=hq, num_kv_heads=hk,
                          head_dim=D, page_size=ps, max_kv=600, causal=causal, window_left=wl,
                          stale="nan", device=gpu)
    plan, ws, k, v, kf, vf, cu_q, cu_k = _dense(pkv, w)
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((w.q.shape[0], hq), float("nan"), dtype=torch.float32, device=gpu)
    pkv.dense_run(plan, w.q, k, v, out, ws, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_dense(w.q.cpu(), k.cpu(), v.cpu(), cu_q, cu_k,
                                          num_qo_heads=hq, num_kv_heads=hk, causal=causal,
                                          window_left=wl)
    compare(out, lse, ref_o, ref_l, f"dense s{seed}")
    p_out, p_lse, _, _ = gpu_run(pkv, w)
    assert torch.equal(out.view(torch.int16), p_out.view(torch.int16)), "dense != paged output bits"
    assert torch.equal(lse.view(torch.int32), p_lse.view(torch.int32)), "dense != paged lse bits"


def test_full_ragged_prefill_dense(pkv, gpu):
    say("case ragged_prefill dense (full size): bit-identical to paged, every element against the oracle")
    w = synth.make_workload("ragged_prefill", device=gpu)
    plan, ws, k, v, kf, vf, cu_q, cu_k = _dense(pkv, w)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.q.shape[0], w.num_qo_heads, dtype=torch.float32, device=gpu)
    pkv.dense_run(plan, w.q, k, v, out, ws, lse=lse)
    p_out, p_lse, _, _ = gpu_run(pkv, w)
    assert torch.equal(out.view(torch.int16), p_out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), p_lse.view(torch.int32))
    ref_o, ref_l = oracle_all(w)
    compare(out, lse, ref_o, ref_l, f"ragged_prefill dense full (all {w.total_q} tokens)", flat=True)
