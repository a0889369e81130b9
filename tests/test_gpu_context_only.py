"""Attention over context-only views on the GPU (kv.plan, context_only_views):
the library's host function drops each row's appended tokens, the plan runs
non-causal over the kept keys, and the result matches the oracle on the same
views.  Covers the prefill tiles (several query blocks and a ragged tail) and
the decode tiles with split-KV (one query per row)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, gpu_run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def _views(pkv, w, seed, one_query):
    rng = np.random.default_rng(seed)
    tc = np.array([rng.integers(0, min(int(n), 96)) for n in w.kv_len])
    if one_query:
        spans = np.ones(w.batch, dtype=np.int64)
    else:
        spans = np.array([rng.integers(1, min(int(n) - int(t), 150) + 1)
                          for n, t in zip(w.kv_len, tc)])
    ptr, idx, lpl, qo = pkv.context_only_views(w.page_size, w.kv_indptr, w.kv_indices,
                                               w.last_page_len, tc, spans)
    g = torch.Generator(device=w.q.device).manual_seed(seed)
    q = torch.randn(int(qo[-1]), w.num_qo_heads, w.head_dim, generator=g,
                    device=w.q.device).to(torch.bfloat16)
    kept = w.kv_len - tc
    return dataclasses.replace(w, kind="decode" if one_query else "prefill", causal=False,
                               kv_len=kept, q_len=spans, qo_indptr=qo, kv_indptr=ptr,
                               kv_indices=idx, last_page_len=lpl, q=q)


def _oracle(v):
    vc = v.to("cpu")
    return oracle.attention(vc.q, vc.cache, v.page_size, v.kv_indptr, v.kv_indices,
                            v.last_page_len, num_qo_heads=v.num_qo_heads,
                            num_kv_heads=v.num_kv_heads, qo_indptr=v.qo_indptr, causal=False,
                            window_left=-1)


@pytest.mark.parametrize("seed,D,hq,hk,ps", [(600, 128, 8, 2, 16), (601, 64, 8, 8, 4),
                                             (602, 128, 16, 4, 32)])
def test_context_only_prefill(pkv, gpu, seed, D, hq, hk, ps):
    say(f"case context_only prefill seed={seed} D={D} Hq={hq} Hk={hk} ps={ps}")
    w = synth.random_case(seed, kind="prefill", batch=6, num_qo_heads=hq, num_kv_heads=hk,
                          head_dim=D, page_size=ps, max_kv=700, stale="nan", device=gpu)
    v = _views(pkv, w, seed, one_query=False)
    out, lse, plan, _ = gpu_run(pkv, v)
    ref_o, ref_l = _oracle(v)
    compare(out, lse, ref_o, ref_l, f"context_only prefill s{seed}")


@pytest.mark.parametrize("seed,split", [(610, False), (611, True)])
def test_context_only_decode(pkv, gpu, seed, split):
    say(f"case context_only decode seed={seed} split={split}")
    w = synth.random_case(seed, kind="decode", batch=9, num_qo_heads=32, num_kv_heads=8,
                          head_dim=128, page_size=16, max_kv=900, stale="nan", device=gpu)
    v = _views(pkv, w, seed, one_query=True)
    kw = dict(num_cus=64, decode_waves_per_cu=16, decode_min_chunk_pages=1) if split else {}
    out, lse, plan, _ = gpu_run(pkv, v, **kw)
    if split:
        assert len(plan.merges()) > 0
    ref_o, ref_l = _oracle(v)
    compare(out, lse, ref_o, ref_l, f"context_only decode s{seed}")
