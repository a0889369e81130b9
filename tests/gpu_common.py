"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compute the oracle for the same bytes on the CPU."""
import sys

import numpy as np
import torch

import oracle

# Tolerances for bf16 inputs with fp32 accumulation.  The output tensor is
# bf16, so the bound on out is OUT_TOL on the computation plus the output's own
# rounding, half a bf16 ulp of the reference (at most 1e-3 below |ref| = 0.5).
OUT_TOL = 1e-2
LSE_TOL = 1e-3   # max |lse - ref|


def half_ulp_bf16(x):
    """Half a bf16 ulp at |x| (bf16 keeps 8 significant bits): the error of
    rounding the exact result to the bf16 output itself."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


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


def oracle_rows(w, rows, tokens=None, cache=None):
    """Oracle output for selected rows, gathering only their pages to the host.
    Returns {r: (out [n, Hq, D], lse [n, Hq])}."""
    cache = w.cache if cache is None else cache
    res = {}
    for r in rows:
        pages = w.kv_indices[w.kv_indptr[r]:w.kv_indptr[r + 1]]
        sub = cache[torch.from_numpy(pages.astype(np.int64)).to(cache.device)].cpu()
        q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        sub_q = w.q[q0:q1].cpu()
        toks = None if tokens is None else {0: tokens[r]}
        one = oracle.attention_rows(sub_q, sub, w.page_size, np.array([0, len(pages)]),
                                    np.arange(len(pages)), w.last_page_len[r:r + 1],
                                    num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                    qo_indptr=np.array([0, q1 - q0]), causal=w.causal,
                                    window_left=w.window_left, tokens=toks)
        res[r] = one[0]
    return res


def compare(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    """Assert the documented tolerances; returns (max out err, max lse err)."""
    o = out_gpu.float().double().cpu().numpy() if hasattr(out_gpu, "cpu") else out_gpu
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - out_ref)
    eo = float(np.max(err)) if o.size else 0.0
    excess = float(np.max(err - OUT_TOL - half_ulp_bf16(out_ref))) if o.size else -1.0
    el = 0.0
    if lse_gpu is not None:
        l = lse_gpu.double().cpu().numpy() if hasattr(lse_gpu, "cpu") else lse_gpu
        assert np.all(np.isfinite(l)), f"{what}: non-finite lse"
        el = float(np.max(np.abs(l - lse_ref))) if l.size else 0.0
    say(f"  {what}: max|out-ref|={eo:.3e} max|lse-ref|={el:.3e} max|ref|={np.max(np.abs(out_ref)) if o.size else 0:.2f}")
    assert excess <= 0, f"{what}: out error {eo} beyond 1e-2 + half a bf16 ulp of the reference"
    assert el <= LSE_TOL, f"{what}: lse error {el}"
    return eo, el
