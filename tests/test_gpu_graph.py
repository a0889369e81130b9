"""Graph-static plans under stream capture (attn.wrappers: static buffers for
graph capture; the replayed graph reads the plan the last upload put in the
workspace).

One graph holding append_kv + run is captured on the first step and replayed
for later steps whose page tables, lengths and row counts differ.  Between the
replays the program re-plans, uploads eagerly and synchronises.  Every replay
is compared with eager calls of the same plan on the same inputs (bit for bit,
outputs and the appended cache) and with the oracle (tolerances).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, say

pytestmark = pytest.mark.gpu

POOL = 2400


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _step(kind, seed, gpu):
    rng = np.random.default_rng(seed)
    if kind == "decode":
        B = int(rng.integers(3, 17))
        kv = rng.integers(1, 1500, size=B)
        ql = np.ones(B, dtype=np.int64)
        hq, hk, d, ps = 32, 8, 128, 16
    else:  # mixed: decode rows and up to 3 prompt rows
        B = int(rng.integers(4, 13))
        kv = rng.integers(1, 700, size=B)
        ql = np.ones(B, dtype=np.int64)
        for r in rng.choice(B, size=3, replace=False):
            ql[r] = rng.integers(2, min(int(kv[r]), 200) + 1) if kv[r] >= 2 else 1
        hq, hk, d, ps = 16, 4, 64, 16
    return synth.from_lengths(f"graph{seed}", kind, kv, ql, num_qo_heads=hq, num_kv_heads=hk,
                              head_dim=d, page_size=ps, pool_pages=POOL, seed=seed, device=gpu,
                              stale="nan", new_tokens=True, max_prefill_rows=3)


@pytest.mark.parametrize("kind,seeds", [("decode", [900, 901, 902, 903]),
                                        ("mixed", [910, 911, 912, 913])])
def test_captured_step_replays_with_new_plans(pkv, gpu, kind, seeds):
    steps = [_step(kind, s, gpu) for s in seeds]
    w0 = steps[0]
    hq, hk, d = w0.num_qo_heads, w0.num_kv_heads, w0.head_dim
    B_cap, T_cap = 16, 640
    params = pkv.plan_params(kind, num_qo_heads=hq, num_kv_heads=hk, head_dim=d,
                             page_size=w0.page_size, max_pages=POOL, max_prefill_rows=3,
                             static_max_batch=B_cap, static_max_tokens=T_cap,
                             static_max_page_entries=POOL,
                             # small tiles budget so that rows split and merges run
                             num_cus=32, decode_waves_per_cu=4, decode_min_chunk_pages=1)
    qo = lambda w: None if kind == "decode" else w.qo_indptr
    plan = pkv.plan_create(params, qo(w0), w0.kv_indptr, w0.kv_indices, w0.last_page_len)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=gpu)
    cache = torch.empty_like(w0.cache)
    q = torch.zeros(T_cap, hq, d, dtype=torch.bfloat16, device=gpu)
    k_new = torch.zeros(T_cap, hk, d, dtype=torch.bfloat16, device=gpu)
    v_new = torch.zeros_like(k_new)
    out = torch.zeros_like(q)
    lse = torch.zeros(T_cap, hq, dtype=torch.float32, device=gpu)

    def load(w):
        T = w.total_q
        cache.copy_(w.cache)
        q[:T].copy_(w.q)
        k_new[:T].copy_(w.k_new)
        v_new[:T].copy_(w.v_new)

    def eager():
        pkv.append_kv(plan, k_new, v_new, cache, ws)
        pkv.run(plan, q, cache, out, ws, lse=lse)

    # warm up (code objects load on first launch), then capture on the first step
    load(w0)
    pkv.plan_upload(plan, ws)
    eager()
    torch.cuda.synchronize()
    load(w0)
    pkv.plan_upload(plan, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eager()
    torch.cuda.synchronize()

    for i, w in enumerate(steps):
        say(f"case graph {kind} step {i} seed={seeds[i]} rows={w.batch} tokens={w.total_q}")
        pkv.plan_update(plan, qo(w), w.kv_indptr, w.kv_indices, w.last_page_len)
        load(w)
        pkv.plan_upload(plan, ws)
        g.replay()
        torch.cuda.synchronize()
        T = w.total_q
        g_out, g_lse, g_cache = out[:T].clone(), lse[:T].clone(), cache.clone()
        # the same plan, eagerly, on the same inputs
        out.fill_(0)
        lse.fill_(0)
        load(w)
        eager()
        torch.cuda.synchronize()
        assert torch.equal(g_out.view(torch.int16), out[:T].view(torch.int16)), "graph != eager out"
        assert torch.equal(g_lse.view(torch.int32), lse[:T].view(torch.int32)), "graph != eager lse"
        assert torch.equal(g_cache.view(torch.int16), cache.view(torch.int16)), "graph != eager cache"
        # the oracle on the appended cache
        slots = oracle.write_slots(w.page_size, w.kv_indptr, w.kv_indices, w.last_page_len,
                                   qo_indptr=qo(w))
        app = oracle.apply_append(_bits(w.cache), slots, _bits(w.k_new), _bits(w.v_new),
                                  w.page_size)
        assert np.array_equal(_bits(g_cache), app)
        ref_o, ref_l = oracle.attention(w.q.cpu(), g_cache.cpu(), w.page_size, w.kv_indptr,
                                        w.kv_indices, w.last_page_len, num_qo_heads=hq,
                                        num_kv_heads=hk, qo_indptr=qo(w), causal=True,
                                        window_left=-1)
        compare(g_out, g_lse, ref_o, ref_l, f"graph {kind} step {i}")

    # an empty step: every captured kernel runs and finds no work
    say(f"case graph {kind} empty step")
    empty = np.zeros(0, dtype=np.int32)
    pkv.plan_update(plan, None if kind == "decode" else np.zeros(1, np.int32),
                    np.zeros(1, np.int32), empty, empty)
    pkv.plan_upload(plan, ws)
    out.fill_(7.0)
    before = cache.clone()
    g.replay()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and torch.equal(cache.view(torch.int16), before.view(torch.int16))
