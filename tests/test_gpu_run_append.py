"""pkv_run_append and repeated runs of one upload.

- pkv_run_append leaves the cache and the outputs bit-identical to
  pkv_append_kv followed by pkv_run, and both match the oracle on the appended
  cache (decode with and without split-KV, prefill and mixed plans);
- one upload serves repeated runs with identical results.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, params_for, say

pytestmark = pytest.mark.gpu

SPLIT = dict(num_cus=64, decode_waves_per_cu=16, decode_min_chunk_pages=1)


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def _oracle(w, cache):
    return oracle.attention(w.q.cpu(), cache.cpu(), w.page_size, w.kv_indptr, w.kv_indices,
                            w.last_page_len, num_qo_heads=w.num_qo_heads,
                            num_kv_heads=w.num_kv_heads,
                            qo_indptr=None if w.kind == "decode" else w.qo_indptr,
                            causal=w.causal, window_left=w.window_left)


def _plan(pkv, w, **kw):
    qo = None if w.kind == "decode" else w.qo_indptr
    plan = pkv.plan_create(params_for(pkv, w, **kw), qo, w.kv_indptr, w.kv_indices, w.last_page_len)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=w.q.device)
    pkv.plan_upload(plan, ws)
    return plan, ws


def _outs(w):
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((w.q.shape[0], w.num_qo_heads), float("nan"), dtype=torch.float32,
                     device=w.q.device)
    return out, lse


@pytest.mark.parametrize("seed,kind,D,hq,hk,ps,split", [
    (400, "decode", 128, 32, 8, 16, True),
    (401, "decode", 64, 8, 8, 32, False),
    (402, "decode", 128, 16, 2, 4, True),
    (403, "prefill", 64, 8, 2, 16, False),
    (404, "mixed", 128, 16, 4, 16, True),
])
def test_run_append_equals_append_then_run(pkv, gpu, seed, kind, D, hq, hk, ps, split):
    say(f"case run_append seed={seed} kind={kind} D={D} Hq={hq} Hk={hk} ps={ps} split={split}")
    if kind == "mixed":  # decode rows (one query) among prompt rows
        kv = np.array([300, 17, 520, 64, 1, 450, 33, 200, 90])
        ql = np.array([1, 1, 40, 1, 1, 90, 2, 1, 0])
        w = synth.from_lengths(f"mixed{seed}", "mixed", kv, ql, num_qo_heads=hq, num_kv_heads=hk,
                               head_dim=D, page_size=ps, seed=seed, stale="nan", new_tokens=True,
                               max_prefill_rows=4, device=gpu)
    else:
        w = synth.random_case(seed, kind=kind, batch=9, num_qo_heads=hq, num_kv_heads=hk,
                              head_dim=D, page_size=ps, max_kv=600, new_tokens=True, stale="nan",
                              device=gpu)
    kw = SPLIT if split else {}
    cache_a, cache_b = w.cache.clone(), w.cache.clone()
    pa, wsa = _plan(pkv, w, **kw)
    oa, la = _outs(w)
    pkv.append_kv(pa, w.k_new, w.v_new, cache_a, wsa)
    pkv.run(pa, w.q, cache_a, oa, wsa, lse=la)
    pb, wsb = _plan(pkv, w, **kw)
    ob, lb = _outs(w)
    pkv.run_append(pb, w.q, w.k_new, w.v_new, cache_b, ob, wsb, lse=lb)
    torch.cuda.synchronize()
    if split and kind != "prefill":
        assert len(pb.merges()) > 0
    bits = lambda t: t.cpu().contiguous().view(torch.int16)
    assert torch.equal(bits(cache_a), bits(cache_b)), "caches differ"
    assert torch.equal(bits(oa), bits(ob)) and torch.equal(la, lb), "outputs differ"
    ref_o, ref_l = _oracle(w, cache_a)
    compare(ob, lb, ref_o, ref_l, f"run_append s{seed}")


def test_one_upload_serves_repeated_runs(pkv, gpu):
    say("case one upload, three runs")
    w = synth.random_case(420, kind="decode", batch=9, num_qo_heads=32, num_kv_heads=8,
                          head_dim=128, page_size=16, max_kv=900, device=gpu)
    plan, ws = _plan(pkv, w, **SPLIT)
    assert len(plan.merges()) > 0
    res = []
    for _ in range(3):
        out, lse = _outs(w)
        pkv.run(plan, w.q, w.cache, out, ws, lse=lse)
        res.append((out, lse))
    torch.cuda.synchronize()
    for out, lse in res[1:]:
        assert torch.equal(out, res[0][0]) and torch.equal(lse, res[0][1])
    ref_o, ref_l = _oracle(w, w.cache)
    compare(res[0][0], res[0][1], ref_o, ref_l, "repeated runs")
