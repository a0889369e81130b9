"""Re-planning while earlier steps are still queued (kv.plan PinnedIndexRing:
a pinned buffer is reused only after its copy finished; attn.dense
force_double_buffer: plan N+1 must not overwrite what step N still reads).

Several plan_update + upload + run steps with different page tables are queued
on one stream behind two full-size long-context decode runs, with no host
synchronisation in between and no forced wait: the only thing keeping a step's
staged metadata intact until its upload kernel has read it is the staging
ring's completion-flag guard.  Each step has its own output buffer and is
checked against the oracle for its own page table.
"""
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


def _table(w, rows):
    """Page table of the given rows of w (in that order)."""
    npages = np.array([w.kv_indptr[r + 1] - w.kv_indptr[r] for r in rows], dtype=np.int64)
    indptr = np.zeros(len(rows) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npages)
    indices = np.concatenate([w.row_pages(r) for r in rows]).astype(np.int32)
    lpl = w.last_page_len[rows].astype(np.int32)
    return indptr, indices, lpl


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_replans_queued_behind_long_work(pkv, gpu, kind):
    say(f"case staging ring: 5 {kind} re-plans queued behind two long_decode runs, no host sync")
    H, Hk, D, ps = 32, 8, 128, 16
    pool = synth.random_case(77, kind="decode", batch=24, num_qo_heads=H, num_kv_heads=Hk,
                             head_dim=D, page_size=ps, max_kv=1500, stale="nan", device=gpu)
    rng = np.random.default_rng(78)
    steps = []
    for k in range(5):
        rows = rng.permutation(pool.batch)[: 6 + 3 * k]
        indptr, indices, lpl = _table(pool, rows)
        kvl = (indptr[1:] - indptr[:-1] - 1) * ps + lpl
        if kind == "decode":
            qo = np.arange(len(rows) + 1, dtype=np.int32)
        else:
            ql = np.minimum(kvl, rng.integers(1, 200, size=len(rows)))
            qo = np.zeros(len(rows) + 1, dtype=np.int32)
            qo[1:] = np.cumsum(ql)
        g = torch.Generator(device=gpu).manual_seed(500 + k)
        q = torch.randn((int(qo[-1]), H, D), generator=g, device=gpu).to(torch.bfloat16)
        steps.append(dict(indptr=indptr, indices=indices, lpl=lpl, qo=qo, q=q))
    params = pkv.plan_params(kind, num_qo_heads=H, num_kv_heads=Hk, head_dim=D, page_size=ps,
                             max_pages=pool.max_pages)
    # workspace for the largest step (sizes come from host-only plans)
    need = 0
    for st in steps:
        tmp = pkv.plan_create(params, None if kind == "decode" else st["qo"], st["indptr"],
                              st["indices"], st["lpl"])
        need = max(need, tmp.ws_bytes)
        del tmp
    ws = torch.empty(need, dtype=torch.uint8, device=gpu)
    outs = [torch.full_like(st["q"], float("nan")) for st in steps]
    lses = [torch.full((st["q"].shape[0], H), float("nan"), dtype=torch.float32, device=gpu)
            for st in steps]

    # long work ahead on the same stream
    lw = synth.make_workload("long_decode", device=gpu)
    lp = pkv.plan_create(pkv.plan_params("decode", num_qo_heads=32, num_kv_heads=8, head_dim=128,
                                         page_size=16, max_pages=lw.max_pages),
                         None, lw.kv_indptr, lw.kv_indices, lw.last_page_len)
    lws = torch.empty(lp.ws_bytes, dtype=torch.uint8, device=gpu)
    lout = torch.empty_like(lw.q)
    torch.cuda.synchronize()

    # Grow both staging buffers to the largest step first: a buffer that must
    # grow is freed and re-allocated, and freeing page-locked memory waits for
    # the device, which would drain the queue this test builds.
    plan = None
    for st in steps + steps:
        qo = None if kind == "decode" else st["qo"]
        if plan is None:
            plan = pkv.plan_create(params, qo, st["indptr"], st["indices"], st["lpl"])
        else:
            pkv.plan_update(plan, qo, st["indptr"], st["indices"], st["lpl"])
        pkv.plan_upload(plan, ws)
        torch.cuda.synchronize()
    warm = plan.upload_stats()

    pkv.plan_upload(lp, lws)
    pkv.run(lp, lw.q, lw.cache, lout, lws)
    pkv.run(lp, lw.q, lw.cache, lout, lws)
    for k, st in enumerate(steps):
        qo = None if kind == "decode" else st["qo"]
        pkv.plan_update(plan, qo, st["indptr"], st["indices"], st["lpl"])
        pkv.plan_upload(plan, ws)
        pkv.run(plan, st["q"], pool.cache, outs[k], ws, lse=lses[k])
    end = plan.upload_stats()
    torch.cuda.synchronize()
    stats = {k: end[k] - warm[k] for k in end}
    say(f"  upload stats of the queued steps: {stats}")
    assert stats["uploads"] == len(steps)
    assert stats["waits"] >= 1, "no upload found its staging buffer busy: the guard was not exercised"

    cache_host = pool.cache.cpu()
    for k, st in enumerate(steps):
        ref_o, ref_l = oracle.attention(st["q"].cpu(), cache_host, ps, st["indptr"], st["indices"],
                                        st["lpl"], num_qo_heads=H, num_kv_heads=Hk,
                                        qo_indptr=None if kind == "decode" else st["qo"],
                                        causal=True, window_left=-1)
        compare(outs[k], lses[k], ref_o, ref_l, f"staging {kind} step {k}")
