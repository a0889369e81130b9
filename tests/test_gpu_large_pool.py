"""Pages past the 4 GiB mark of a layer slice: every kernel addresses a page
with a 64-bit byte offset (page id x page bytes).  Each case's pages are
moved to the top of a pool of more than 4 GiB and the run is compared with
the oracle on the original (small) pool, which holds the same logical K/V."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


CASES = [
    # (kind, Hq, Hk, D, page_size, window)
    ("prefill", 32, 8, 128, 16, -1),
    ("prefill", 16, 2, 64, 32, 200),
    ("decode", 32, 8, 128, 16, -1),
    ("mixed", 16, 16, 64, 32, 300),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-D{c[3]}-g{c[1]//c[2]}-ps{c[4]}")
def test_pages_above_4gib(pkv, gpu, case):
    kind, hq, hk, D, ps, wl = case
    say(f"case large pool {kind} Hq={hq} Hk={hk} D={D} ps={ps} window={wl}")
    rng = np.random.default_rng(61)
    if kind == "mixed":
        kv = np.concatenate([rng.integers(50, 900, size=6), [700, 1100]])
        ql = np.concatenate([np.ones(6, np.int64), [300, 500]])
        order = rng.permutation(len(kv))
        w = synth.from_lengths("large_mixed", "mixed", kv[order], ql[order], num_qo_heads=hq,
                               num_kv_heads=hk, head_dim=D, page_size=ps, window_left=wl,
                               rng=rng, seed=61, device=gpu, stale="nan", max_prefill_rows=2)
    else:
        w = synth.random_case(62, kind=kind, batch=6, num_qo_heads=hq, num_kv_heads=hk, head_dim=D,
                              page_size=ps, max_kv=900, window_left=wl, stale="nan", device=gpu)
    page_bytes = 2 * ps * hk * D * 2
    first_high = -(-(4 << 30) // page_bytes)            # first page id at or past 4 GiB
    n_used = len(w.kv_indices)
    pool = first_high + n_used + 7
    assert pool * page_bytes > (4 << 30) + page_bytes
    big = torch.full((pool, 2, ps, hk, D), float("nan"), dtype=torch.bfloat16, device=gpu)
    new_ids = (first_high + rng.permutation(n_used)).astype(np.int32)
    big[torch.from_numpy(new_ids.astype(np.int64)).to(gpu)] = \
        w.cache[torch.from_numpy(w.kv_indices.astype(np.int64)).to(gpu)]
    params = pkv.plan_params(kind, num_qo_heads=hq, num_kv_heads=hk, head_dim=D, page_size=ps,
                             max_pages=pool, window_left=wl, max_prefill_rows=w.max_prefill_rows)
    qo = None if kind == "decode" else w.qo_indptr
    plan = pkv.plan_create(params, qo, w.kv_indptr, new_ids, w.last_page_len)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=gpu)
    pkv.plan_upload(plan, ws)
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((w.q.shape[0], hq), float("nan"), dtype=torch.float32, device=gpu)
    pkv.run(plan, w.q, big, out, ws, lse=lse)
    torch.cuda.synchronize()
    del big
    ref_o, ref_l = oracle.attention(w.q.cpu(), w.cache.cpu(), ps, w.kv_indptr, w.kv_indices,
                                    w.last_page_len, num_qo_heads=hq, num_kv_heads=hk,
                                    qo_indptr=qo, causal=True, window_left=wl)
    compare(out, lse, ref_o, ref_l, f"large pool {kind} D{D}")
