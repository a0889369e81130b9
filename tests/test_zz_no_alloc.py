"""pkv_run_noalloc: upload + run with the library's static per-GPU workspace,
for callers that cannot allocate.  Checked against the existing entry points
(pkv_plan_upload + pkv_run on a caller workspace) bit for bit and against the
oracle, on two calls in a row, the second with a smaller input."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, say


@pytest.fixture(scope="module")
def pkv_cpu():
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def test_oversized_plan_is_rejected_before_any_device_call(pkv_cpu):
    # a plan whose workspace (split-KV partials) exceeds the static array
    w = synth.make_workload("long_decode", layout_only=True)
    p = pkv_cpu.plan_create(pkv_cpu.plan_params("decode", num_qo_heads=32, num_kv_heads=8,
                                                head_dim=128, page_size=16, max_pages=w.max_pages,
                                                num_cus=4096, decode_waves_per_cu=16,
                                                decode_min_chunk_pages=1),
                            None, w.kv_indptr, w.kv_indices, w.last_page_len)
    assert p.ws_bytes > pkv_cpu.noalloc_capacity()
    st = pkv_cpu._lib.pkv_run_noalloc(p.handle, None, None, None, None, None)
    assert st == pkv_cpu.E_CAPACITY
    assert "static workspace" in pkv_cpu._lib.pkv_last_error().decode()


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def _rows(w, rows):
    npages = np.array([w.kv_indptr[r + 1] - w.kv_indptr[r] for r in rows], dtype=np.int64)
    indptr = np.zeros(len(rows) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npages)
    indices = np.concatenate([w.row_pages(r) for r in rows]).astype(np.int32)
    qo = np.zeros(len(rows) + 1, dtype=np.int32)
    qo[1:] = np.cumsum(w.q_len[rows])
    q = torch.cat([w.q[int(w.qo_indptr[r]):int(w.qo_indptr[r + 1])] for r in rows])
    return qo, indptr, indices, w.last_page_len[rows].astype(np.int32), q


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["gqa_decode", "mixed_window"])
def test_noalloc_matches_upload_and_run(pkv, gpu, name):
    say(f"case run_noalloc on {name}: all rows, then a smaller step")
    w = synth.make_workload(name, device=gpu, stale="nan")
    big = list(range(w.batch))
    small = [r for r in range(w.batch) if r % 3 == 1]
    if name == "mixed_window":  # keep two prompt rows in the smaller step
        pr = [r for r in big if w.q_len[r] > 1]
        small = sorted(set(small) | set(pr[:2]))
    params = pkv.plan_params(w.kind, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                             head_dim=w.head_dim, page_size=w.page_size, max_pages=w.max_pages,
                             causal=w.causal, window_left=w.window_left,
                             max_prefill_rows=w.max_prefill_rows)
    plan = None
    for k, rows in enumerate([big, small]):
        qo, indptr, indices, lpl, q = _rows(w, rows)
        qo_arg = None if w.kind == "decode" else qo
        if plan is None:
            plan = pkv.plan_create(params, qo_arg, indptr, indices, lpl)
        else:
            pkv.plan_update(plan, qo_arg, indptr, indices, lpl)
        # the existing entry points, on a caller workspace (this also sizes the
        # plan's staging buffers on the first step)
        ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=gpu)
        pkv.plan_upload(plan, ws)
        # with the plan's own timing on, pkv_run records its launches and
        # pkv_run_noalloc records none (its events would be created on first use)
        pkv.timing_enable(plan)
        out_ref = torch.full_like(q, float("nan"))
        lse_ref = torch.full((q.shape[0], w.num_qo_heads), float("nan"), device=gpu)
        pkv.run(plan, q, w.cache, out_ref, ws, lse=lse_ref)
        assert sum(n for _, n in pkv.timing_read(plan).values()) > 0
        # the static workspace
        out = torch.full_like(q, float("nan"))
        lse = torch.full((q.shape[0], w.num_qo_heads), float("nan"), device=gpu)
        pkv.run_noalloc(plan, q, w.cache, out, lse=lse)
        torch.cuda.synchronize()
        assert sum(n for _, n in pkv.timing_read(plan).values()) == 0
        pkv.timing_enable(plan, False)
        say(f"  step {k}: {len(rows)} rows, {q.shape[0]} queries, workspace {plan.ws_bytes} bytes")
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), "out bits differ"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), "lse bits differ"
        ref_o, ref_l = oracle.attention(q.cpu(), w.cache.cpu(), w.page_size, indptr, indices, lpl,
                                        num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                        qo_indptr=qo_arg, causal=w.causal,
                                        window_left=w.window_left)
        compare(out, lse, ref_o, ref_l, f"run_noalloc {name} step {k}", flat=True)


@pytest.mark.gpu
def test_noalloc_needs_sized_staging(pkv, gpu):
    say("case run_noalloc on a plan never uploaded: staging too small, no launch")
    w = synth.random_case(900, kind="decode", batch=5, num_qo_heads=8, num_kv_heads=2,
                          head_dim=128, page_size=16, max_kv=300, device=gpu)
    plan = pkv.plan_create(pkv.plan_params("decode", num_qo_heads=8, num_kv_heads=2, head_dim=128,
                                           page_size=16, max_pages=w.max_pages),
                           None, w.kv_indptr, w.kv_indices, w.last_page_len)
    out = torch.zeros_like(w.q)
    with pytest.raises(pkv.PkvError) as e:
        pkv.run_noalloc(plan, w.q, w.cache, out)
    assert e.value.status == pkv.E_CAPACITY
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)) == 0
