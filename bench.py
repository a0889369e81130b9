"""Benchmark: batched attention over a paged KV cache on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config NAME] [--no-cpu-baseline]
                    [--no-secondary] [--no-ceilings]

A step is one pass of the whole hot path over one batch of synthetic input that
is already resident in HBM: host re-plan of the page table (pkv_plan_update),
upload of the plan metadata, KV append of this step's token (decode workloads),
and attention (decode + split-KV merge, prefill, or both for the mixed step).

The headline workload is batched GQA decode with append: 128 requests,
32 query heads over 8 KV heads, head_dim 128, page size 16, kv_len uniform in
[512, 4096], pages drawn from a 40000-page pool.  Its metric is KV bytes read
per second.  The other workloads (long-context split-KV decode, causal ragged
prefill, mixed step with a sliding window) are measured briefly and reported
under "secondary".

Besides the contract fields the line carries, per kernel kind, the mean and
p10 / median / p90 of the event-timed launch durations; the host time of
pkv_plan_update and the device time of the metadata upload, measured apart
from the step; and measured ceilings of this GPU (a 2 GiB device copy, a
bf16 GEMM, a register-only bf16 MFMA loop and a 2 GiB streaming read) as
context for the spec peaks.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published

METRIC = "decode KV-read GB/s (% HBM peak); prefill TFLOP/s (% bf16 MFMA peak)"

# rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch) against a plain copy kernel
# of 1 GiB on this GPU: FETCH_SIZE reads 524288 KiB for 1048576 KiB fetched,
# WRITE_SIZE reads 1048576 KiB for 1048576 KiB written.
FETCH_SCALE = 2.0
WRITE_SCALE = 1.0
CSRC = os.path.join(ROOT, "paged_kv_attention_plan_amd", "csrc")
# the files whose text makes each kernel (its launch file and its device code)
KERNEL_SOURCE = {"decode_kernel": ["decode.hip", "decode_body.cuh", "common.cuh"],
                 "prefill_kernel": ["prefill.hip", "prefill_body.cuh", "common.cuh"],
                 "merge_kernel": ["merge_append.hip", "common.cuh"],
                 "append_kernel": ["merge_append.hip", "common.cuh"]}
# oracle seconds each workload's CPU baseline may spend (about 30 s in all)
CPU_BUDGET_S = {"tiny_decode": 2.0, "gqa_decode": 6.0, "long_decode": 6.0, "ragged_prefill": 8.0,
                "mixed_window": 8.0}

DESCR = {
    "tiny_decode": "tiny decode: 4 requests, Hq 4 / Hk 2, D 64, page 16, kv_len U[1,100]",
    "gqa_decode": "batched GQA decode + append: 128 requests, Hq 32 / Hk 8, D 128, page 16, "
                  "kv_len U[512,4096], 40000-page pool",
    "long_decode": "long-context split-KV decode: 8 requests, Hq 32 / Hk 8, D 128, page 16, "
                   "kv_len U[32768,131072]",
    "ragged_prefill": "causal ragged prefill: 16 requests, q_len U[128,2048], prefix U[0,4096], "
                      "Hq 32 / Hk 8, D 128, page 16",
    "mixed_window": "mixed step, window 4096: 256 decode rows (kv_len U[256,8192]) + 4 prompt rows "
                    "(1024 on 2048 prefix), Hq 16 / Hk 16, D 64, page 32",
    "gqa_decode_context_only": "context-only decode over the gqa_decode rows: each row's appended "
                               "token dropped by context_only_views, one query per row attending "
                               "to the stored kv_len - 1 keys",
    "tiny_decode_graph": "graph-static mode on the tiny decode rows (4 requests, Hq 4 / Hk 2, D 64, "
                         "page 16, kv_len U[1,100]): re-plan and upload eagerly, then one replay "
                         "of a captured append + decode + merge",
    "ragged_prefill_dense": "dense [prefix | fresh] mode over the ragged_prefill rows: prefixes "
                            "gathered from the pages once, each step's fresh K/V copied after "
                            "them, one dense varlen pass (contiguous K/V)",
}


def _source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCE[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_of(kernel, workload):
    """HBM bytes per launch from the committed counter record, or None when no
    record exists or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec["bytes_per_launch"] if rec.get("source_sha256") == _source_sha(kernel) else None


def record_traffic(fetch_csv, write_csv, kernel, workload, command):
    """Write profiles/traffic_<kernel>_<workload>.json from the two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch)."""
    import csv

    def mean_of(path, counter):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter]
        return sum(vals) / len(vals), len(vals)

    fk, fn = mean_of(fetch_csv, "FETCH_SIZE")
    wk, wn = mean_of(write_csv, "WRITE_SIZE")
    rec = {"kernel": kernel, "workload": workload, "source_sha256": _source_sha(kernel),
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk, "dispatches": [fn, wn],
           "fetch_scale": FETCH_SCALE, "write_scale": WRITE_SCALE,
           "bytes_per_launch": int(round((fk * FETCH_SCALE + wk * WRITE_SCALE) * 1024)),
           "command": command}
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(path, rec["bytes_per_launch"])


def visible_counts(w):
    """Per query token: number of visible keys (causal, window), in q order."""
    out = np.zeros(w.total_q, dtype=np.int64)
    for r in range(w.batch):
        n, L = int(w.kv_len[r]), int(w.q_len[r])
        q0 = int(w.qo_indptr[r])
        for t in range(L):
            p = n - L + t
            hi = p if w.causal else n - 1
            lo = 0 if w.window_left < 0 else max(0, p - w.window_left)
            out[q0 + t] = hi - lo + 1
    return out


def work_of(w):
    """Algorithmic work.  Decode rows (one query): bytes of visible K and V once
    per KV head, plus q and out.  Prompt rows: 4*D FLOP per visible
    (query token, query head, key)."""
    vis = visible_counts(w)
    is_dec = np.zeros(w.total_q, dtype=bool)
    for r in range(w.batch):
        if w.kind == "decode" or (w.kind == "mixed" and w.q_len[r] == 1):
            is_dec[int(w.qo_indptr[r])] = True
    D, Hq, Hk = w.head_dim, w.num_qo_heads, w.num_kv_heads
    kv_bytes = int(vis[is_dec].sum()) * Hk * D * 2 * 2
    qo_bytes = int(is_dec.sum()) * Hq * D * 2 * 2
    flops = int(vis[~is_dec].sum()) * Hq * 4 * D
    return {"kv_bytes": kv_bytes, "decode_bytes": kv_bytes + qo_bytes, "prefill_flops": flops}


def aux_bytes(plan, w, appended):
    """Algorithmic bytes per launch of the merge (every partial output and LSE
    read once, the merged bf16 output and fp32 LSE written once) and of the
    append (each new K and V row read once and written once)."""
    g, D = w.num_qo_heads // w.num_kv_heads, w.head_dim
    m = plan.merges()
    chunks = int(m["n_chunks"].sum()) if len(m) else 0
    merge = g * (chunks * (D * 4 + 4) + len(m) * (D * 2 + 4))
    append = 2 * 2 * w.total_q * w.num_kv_heads * D * 2 if appended else 0
    return {"merge_kernel": merge, "append_kernel": append}


def aux_block(kt_ms, nbytes, workload):
    """µs distribution, achieved GB/s and counter traffic of one small kernel."""
    res = {}
    for kind, kname in (("merge", "merge_kernel"), ("append", "append_kernel")):
        ts = kt_ms.get(kind) or []
        if not ts or not nbytes[kname]:
            continue
        us = mean_ms(ts) * 1e3
        res[kname] = {"us": stats(ts, 1e3), "bytes_per_launch": nbytes[kname],
                      "achieved_GBps": round(nbytes[kname] / (us * 1e-6) / 1e9, 1),
                      "frac_hbm_peak": round(nbytes[kname] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "traffic": traffic_of(kname, workload)}
    return res


class Runner:
    """Holds the device buffers and the plan for one workload."""

    def __init__(self, name, dev, waves_per_cu=0, min_chunk_pages=0):
        import torch
        import synth
        from paged_kv_attention_plan_amd import pkv
        self.torch, self.pkv = torch, pkv
        self.name = name
        self.graph = name.endswith("_graph")
        if self.graph:
            name = name[:-len("_graph")]
        self.dense = name.endswith("_dense")
        if self.dense:
            name = name[:-len("_dense")]
        self.context_only = name.endswith("_context_only")
        self.w = synth.make_workload(name[:-len("_context_only")] if self.context_only else name,
                                     device=dev)
        if self.context_only:  # every row's last token is this step's
            import dataclasses
            w0 = self.w
            self.views_in = (w0.page_size, w0.kv_indptr, w0.kv_indices, w0.last_page_len,
                             np.ones(w0.batch, np.int32), np.ones(w0.batch, np.int32))
            ptr, idx, lpl, _ = pkv.context_only_views(*self.views_in)
            self.w = dataclasses.replace(w0, kv_len=w0.kv_len - 1, kv_indptr=ptr, kv_indices=idx,
                                         last_page_len=lpl, causal=False)
        w = self.w
        if w.k_new is None and w.kind == "decode":
            g = torch.Generator(device=dev).manual_seed(7)
            shape = (w.total_q, w.num_kv_heads, w.head_dim)
            w.k_new = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
            w.v_new = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
        self.qo = None if w.kind == "decode" else w.qo_indptr
        if self.dense:
            self._init_dense(dev)
            return
        static = dict(static_max_batch=w.batch, static_max_tokens=w.total_q,
                      static_max_page_entries=len(w.kv_indices)) if self.graph else {}
        self.params = pkv.plan_params(w.kind, num_qo_heads=w.num_qo_heads,
                                      num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                      page_size=w.page_size, max_pages=w.max_pages,
                                      causal=w.causal, window_left=w.window_left,
                                      max_prefill_rows=w.max_prefill_rows,
                                      decode_waves_per_cu=waves_per_cu,
                                      decode_min_chunk_pages=min_chunk_pages, **static)
        self.plan = pkv.plan_create(self.params, self.qo, w.kv_indptr, w.kv_indices,
                                    w.last_page_len)
        self.ws = torch.empty(self.plan.ws_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(w.q)
        self.lse = torch.empty(w.total_q, w.num_qo_heads, dtype=torch.float32, device=dev)
        self.append = w.kind == "decode" and name in ("gqa_decode", "tiny_decode")
        self.step_descr = ("context_only_views + plan_update + upload + run (decode + split-KV "
                           "merge)" if self.context_only else
                           "plan_update + upload + append_kv + run (decode + split-KV merge)"
                           if self.append else "plan_update + upload + run")
        if self.graph:
            self.step_descr = ("plan_update + upload (eager) + replay of a captured append_kv + "
                               "run (decode + split-KV merge)")
            self._capture()
        self.work = work_of(w)

    def _init_dense(self, dev):
        """Dense plan over the same rows: row r's prefix is its first
        kv_len - q_len tokens; the step's fresh K/V are the rows' last q_len
        tokens as the pool holds them.  The prefixes are gathered once here."""
        torch, pkv, w = self.torch, self.pkv, self.w
        self.cu_q = w.qo_indptr.astype(np.int32)
        self.cu_k = np.concatenate([[0], np.cumsum(w.kv_len)]).astype(np.int32)
        self.params = pkv.plan_params("dense", num_qo_heads=w.num_qo_heads,
                                      num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                      page_size=w.page_size, max_pages=w.max_pages,
                                      causal=w.causal, window_left=w.window_left)
        self.plan = pkv.dense_plan_create(self.params, self.cu_q, self.cu_k, w.kv_indptr,
                                          w.kv_indices)
        self.ws = torch.empty(self.plan.ws_bytes, dtype=torch.uint8, device=dev)
        flat = []
        for r in range(w.batch):
            n, L = int(w.kv_len[r]), int(w.q_len[r])
            for j in range(n - L, n):
                flat.append(int(w.kv_indices[w.kv_indptr[r] + j // w.page_size]) * w.page_size
                            + j % w.page_size)
        idx = torch.tensor(flat, dtype=torch.int64, device=dev)
        hk, d = w.num_kv_heads, w.head_dim
        self.k_fresh = w.cache[:, 0].reshape(-1, hk, d)[idx].contiguous()
        self.v_fresh = w.cache[:, 1].reshape(-1, hk, d)[idx].contiguous()
        K = int(self.cu_k[-1])
        self.k_dense = torch.empty(K, hk, d, dtype=torch.bfloat16, device=dev)
        self.v_dense = torch.empty_like(self.k_dense)
        pkv.plan_upload(self.plan, self.ws)
        pkv.dense_gather(self.plan, w.cache, self.k_fresh, self.v_fresh, self.k_dense,
                         self.v_dense, self.ws, with_prefix=True)
        self.out = torch.empty_like(w.q)
        self.lse = torch.empty(w.total_q, w.num_qo_heads, dtype=torch.float32, device=dev)
        self.append = False
        self.step_descr = ("dense_plan_update + upload + dense_gather (fresh rows) + dense_run; "
                           "prefixes gathered once before the timed steps")
        self.work = work_of(w)

    def _eager_kernels(self):
        w, pkv = self.w, self.pkv
        if self.append:
            pkv.append_kv(self.plan, w.k_new, w.v_new, w.cache, self.ws)
        pkv.run(self.plan, w.q, w.cache, self.out, self.ws, lse=self.lse)

    def _capture(self):
        """Warm up, then capture the step's kernels (append_kv + run) of the
        graph-static plan; step() replays them after the eager re-plan and
        upload."""
        torch, pkv = self.torch, self.pkv
        pkv.plan_upload(self.plan, self.ws)
        self._eager_kernels()
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            self._eager_kernels()
        torch.cuda.synchronize()

    def gather_prefix_us(self, reps=10):
        """Event-timed µs of one full gather (prefixes from the pages + fresh rows)."""
        pkv, torch = self.pkv, self.torch
        pkv.timing_read(self.plan)
        pkv.timing_enable(self.plan, True)
        ts = []
        for _ in range(reps):
            pkv.dense_gather(self.plan, self.w.cache, self.k_fresh, self.v_fresh, self.k_dense,
                             self.v_dense, self.ws, with_prefix=True)
            ms, n = pkv.timing_read(self.plan)["append"]
            ts.append(ms / n * 1e3)
        pkv.timing_enable(self.plan, False)
        return stats(ts)

    def step(self):
        w, pkv = self.w, self.pkv
        if self.dense:
            pkv.dense_plan_update(self.plan, self.cu_q, self.cu_k, w.kv_indptr, w.kv_indices)
            pkv.plan_upload(self.plan, self.ws)
            pkv.dense_gather(self.plan, None, self.k_fresh, self.v_fresh, self.k_dense,
                             self.v_dense, self.ws, with_prefix=False)
            pkv.dense_run(self.plan, w.q, self.k_dense, self.v_dense, self.out, self.ws,
                          lse=self.lse)
            return
        if self.graph:
            pkv.plan_update(self.plan, self.qo, w.kv_indptr, w.kv_indices, w.last_page_len)
            pkv.plan_upload(self.plan, self.ws)
            self.g.replay()
            return
        if self.context_only:  # the views are re-derived every step, as a serving loop would
            ptr, idx, lpl, _ = pkv.context_only_views(*self.views_in)
            pkv.plan_update(self.plan, self.qo, ptr, idx, lpl)
        else:
            pkv.plan_update(self.plan, self.qo, w.kv_indptr, w.kv_indices, w.last_page_len)
        pkv.plan_upload(self.plan, self.ws)
        if self.append:
            pkv.append_kv(self.plan, w.k_new, w.v_new, w.cache, self.ws)
        pkv.run(self.plan, w.q, w.cache, self.out, self.ws, lse=self.lse)

    def time_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        with no_gc_pause():
            t0 = time.perf_counter()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                self.step()
            e1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall * 1e3 / steps

    def kernel_times(self, steps):
        """Per-launch ms of each kernel kind over `steps` steps, from HIP events
        the library records around its launches on this stream: kind -> list."""
        pkv = self.pkv
        pkv.timing_read(self.plan)  # clear
        pkv.timing_enable(self.plan, True)
        per = {}
        for _ in range(steps):
            self.step()
            for k, (ms, n) in pkv.timing_read(self.plan).items():
                if n:
                    per.setdefault(k, []).append(ms / n)
        pkv.timing_enable(self.plan, False)
        return {k: per.get(k, []) for k in ("append", "decode", "merge", "prefill")}

    def host_times(self, steps):
        """Host µs of plan_update and device µs of the metadata upload (events
        around pkv_plan_upload on this stream), per step."""
        w, pkv, torch = self.w, self.pkv, self.torch
        plan_us, up_us = [], []
        for _ in range(steps):
            t0 = time.perf_counter()
            if self.dense:
                pkv.dense_plan_update(self.plan, self.cu_q, self.cu_k, w.kv_indptr, w.kv_indices)
            else:
                pkv.plan_update(self.plan, self.qo, w.kv_indptr, w.kv_indices, w.last_page_len)
            plan_us.append((time.perf_counter() - t0) * 1e6)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            pkv.plan_upload(self.plan, self.ws)
            e1.record()
            e1.synchronize()
            up_us.append(e0.elapsed_time(e1) * 1e3)
        return {"plan_update_us": stats(plan_us), "upload_us": stats(up_us),
                "upload_bytes": self.plan.info()["meta_bytes"]}


def stats(xs, scale=1.0):
    """mean / p10 / median / p90 of a list (None when empty), times scale."""
    if not xs:
        return None
    a = np.sort(np.asarray(xs, dtype=np.float64)) * scale
    q = lambda f: float(a[min(len(a) - 1, int(round(f * (len(a) - 1))))])
    return {"mean": round(float(a.mean()), 2), "p10": round(q(0.1), 2),
            "median": round(q(0.5), 2), "p90": round(q(0.9), 2), "n": int(len(a))}


def mean_ms(xs):
    return sum(xs) / len(xs) if xs else None


def ceilings(dev):
    """Measured ceilings on this GPU, for context beside the spec peaks: a
    device-to-device copy of 2 GiB (bytes read + written per second) and a
    bf16 8192^3 matrix product (torch / hipBLASLt), each the best of 5."""
    import torch
    n = 1 << 30  # bf16 elements: 2 GiB per buffer
    src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    best = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        best.append(e0.elapsed_time(e1))
    copy_gbs = 2 * src.numel() * 2 / (min(best[1:]) * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev).to(torch.bfloat16).contiguous()
    b = torch.randn(m, m, device=dev).to(torch.bfloat16).contiguous()
    best = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.mm(a, b)
        e1.record()
        e1.synchronize()
        best.append(e0.elapsed_time(e1))
    gemm_tfs = 2 * m ** 3 / (min(best[1:]) * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    res = {"copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tfs, 1),
           "copy": "torch copy_ of 2 GiB, read + write bytes, best of 5",
           "gemm": "torch.mm bf16 8192 x 8192 x 8192, best of 5"}
    res.update(probe_ceilings(dev))
    return res


def probe_ceilings(dev):
    """The two rates the attention kernels are bound by, from the probe
    library built beside libpkv.so: register-only bf16 MFMA loops
    (v_mfma_f32_32x32x16_bf16, 4096 workgroups of 4 waves, 2048 rounds of four
    independent products each; the same with v_mfma_f32_16x16x32_bf16; and that
    one with operands that change between products, with the shader clock
    measured over each) and a streaming read of 2 GiB (512 workgroups
    of 256 threads, four 16-byte non-temporal loads in flight per thread: the
    best of a sweep of launch shapes), each the best of 5 launches after
    warm-up launches that bring the clocks up."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "paged_kv_attention_plan_amd", "libpkv_ceilings.so")
    if not os.path.exists(path):
        return {"probes": "libpkv_ceilings.so not built"}
    lib = ctypes.CDLL(path)
    lib.pkv_ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.pkv_ceiling_mfma16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.pkv_ceiling_mfma16_rot.argtypes = lib.pkv_ceiling_mfma16.argtypes
    lib.pkv_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    blocks, iters, read_blocks = 4096, 2048, 512
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def best_ms(launch, warm=1):
        t = []
        for _ in range(warm + 5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if launch() != 0:
                raise RuntimeError("probe launch failed")
            e1.record(stream)
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return min(t[warm:])

    ms = best_ms(lambda: lib.pkv_ceiling_mfma(ctypes.c_void_p(sink.data_ptr()), blocks, iters, sh),
                 warm=3)
    mfma_tfs = blocks * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    wall_hz = lib.pkv_ceiling_wallclock_khz() * 1e3

    def clock_ghz():  # shader clock over the launches since the last call
        c = clk.tolist()
        clk.zero_()
        return round(c[0] / c[1] * wall_hz / 1e9, 3) if c[1] > 0 and wall_hz > 0 else None

    ms = best_ms(lambda: lib.pkv_ceiling_mfma16(ctypes.c_void_p(sink.data_ptr()),
                                                ctypes.c_void_p(clk.data_ptr()), blocks, iters, sh),
                 warm=3)
    mfma16_tfs = blocks * 4 * iters * 8 * 16384 / (ms * 1e-3) / 1e12
    mfma16_ghz = clock_ghz()
    # changing operands, long enough (about 12 ms a launch) for the clock to settle
    rot_blocks, rot_iters = 2048, 20000
    ms = best_ms(lambda: lib.pkv_ceiling_mfma16_rot(ctypes.c_void_p(sink.data_ptr()),
                                                    ctypes.c_void_p(clk.data_ptr()), rot_blocks,
                                                    rot_iters, sh), warm=1)
    rot_tfs = rot_blocks * 4 * rot_iters * 8 * 16384 / (ms * 1e-3) / 1e12
    rot_ghz = clock_ghz()
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    ms = best_ms(lambda: lib.pkv_ceiling_read(ctypes.c_void_p(src.data_ptr()), nbytes,
                                              ctypes.c_void_p(sink.data_ptr()), read_blocks, sh))
    read_gbs = nbytes / (ms * 1e-3) / 1e9
    del src, sink
    torch.cuda.empty_cache()
    return {"mfma_loop_TFLOPs": round(mfma_tfs, 1), "read_GBps": round(read_gbs, 1),
            "mfma_loop": "register-only v_mfma_f32_32x32x16_bf16 loop, 16384 waves, best of 5",
            "mfma16_loop_TFLOPs": round(mfma16_tfs, 1),
            "mfma16_loop": "the same with v_mfma_f32_16x16x32_bf16 (the prefill kernel's shape), "
                           "8 chains per wave, best of 5",
            "mfma16_loop_clock_GHz": mfma16_ghz,
            "mfma16_rotating_TFLOPs": round(rot_tfs, 1),
            "mfma16_rotating_clock_GHz": rot_ghz,
            "mfma16_rotating": "the 16x16x32 loop with 16 pseudo-random operand pairs per lane taken "
                               "in turn (operands change between products, as on real data), "
                               "8192 waves x 160000 products, best of 5; the clock is s_memtime "
                               "cycles over s_memrealtime ticks",
            "read": "streaming read of 2 GiB, 512 x 256 threads, 4 x 16-byte loads in flight, best of 5"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        blas = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(blas) if blas else 1
    except Exception:
        return 1


def cpu_baseline(runner, budget_s):
    """The oracle, timed on the host over the rows of the same inputs, in
    order, until about budget_s seconds of work (decode rows and prompt rows
    each get half when a workload has both).  Decode rows are reported in GB/s
    of KV read, prompt rows in TFLOP/s; oracle seconds for the whole workload
    are extrapolated from the sample by its share of the work."""
    import torch
    import oracle
    w = runner.w
    vis = visible_counts(w)
    groups = {"decode": [], "prefill": []}
    for r in range(w.batch):
        L = int(w.q_len[r])
        if L == 1 and w.kind in ("decode", "mixed"):
            groups["decode"].append(r)
        elif L > 0:
            groups["prefill"].append(r)
    groups = {k: v for k, v in groups.items() if v}
    res = {}
    for kind, rows in groups.items():
        share = budget_s / len(groups)
        work = lambda r: (int(vis[int(w.qo_indptr[r])]) * w.num_kv_heads * w.head_dim * 4
                          if kind == "decode" else
                          int(vis[int(w.qo_indptr[r]):int(w.qo_indptr[r + 1])].sum())
                          * w.num_qo_heads * 4 * w.head_dim)
        total = sum(work(r) for r in rows)
        done, amount, elapsed = 0, 0, 0.0
        for r in rows:
            pages = w.kv_indices[w.kv_indptr[r]:w.kv_indptr[r + 1]]
            sub = w.cache[torch.from_numpy(pages.astype(np.int64)).to(w.cache.device)].cpu()
            q0, q1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
            sub_q = w.q[q0:q1].cpu()
            t0 = time.perf_counter()
            oracle.attention_rows(sub_q, sub, w.page_size, np.array([0, len(pages)]),
                                  np.arange(len(pages)), w.last_page_len[r:r + 1],
                                  num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                  qo_indptr=np.array([0, q1 - q0]), causal=w.causal,
                                  window_left=w.window_left)
            elapsed += time.perf_counter() - t0
            amount += work(r)
            done += 1
            if elapsed >= share:
                break
        unit = "GB/s" if kind == "decode" else "TFLOP/s"
        value = amount / elapsed / (1e9 if kind == "decode" else 1e12)
        res[kind] = {"value": round(value, 6), "unit": unit, "oracle_s": round(elapsed, 2),
                     "rows": f"{done} of {len(rows)}",
                     "oracle_s_whole_workload_est": round(elapsed * total / max(amount, 1), 1)}
    return {"cores": int(blas_threads()), "kind": "oracle", "float": "float64 numpy",
            **res}


def headline_cpu_baseline(cb, unit, name):
    """The contract's cpu_baseline object from a cpu_baseline() result."""
    part = cb["decode" if unit == "GB/s" else "prefill"]
    return {"value": part["value"], "unit": part["unit"], "cores": cb["cores"], "kind": "oracle",
            "sample": f"{name}: first {part['rows']} requests of the same seeded input, every "
                      f"query head (float64 numpy), {part['oracle_s']} s; about "
                      f"{part['oracle_s_whole_workload_est']} s for the whole workload"}


@contextlib.contextmanager
def no_gc_pause():
    """Python's cycle collector off inside a timed loop: a full collection over
    the many objects alive by the later workloads takes tens of milliseconds,
    during which the host issues nothing and the GPU idles.  (Nothing is
    collected here: that would change which memory later workloads reuse.)"""
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


def prefill_roofline(kt_ms, flops, workload):
    """The roofline object of the prefill kernel from its event-timed launches."""
    ts = kt_ms["prefill"]
    pms = mean_ms(ts)
    achieved = flops / (pms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
            "traffic": traffic_of("prefill_kernel", workload), "kernel": "prefill_kernel",
            "kernel_us": round(pms * 1e3, 2), "kernel_us_dist": stats(ts, 1e3),
            "flops_per_launch": flops, "workload": workload}


def secondary(name, dev, steps, warmup, with_cpu=False):
    r = Runner(name, dev)
    ms, _ = r.time_steps(steps, warmup)
    if r.graph:  # no per-kernel events inside a replay: compare whole steps with eager ones
        e = Runner(name[:-len("_graph")], dev)
        e_ms, _ = e.time_steps(steps, warmup)
        return {"workload": DESCR[name], "ms_per_step": round(ms, 4),
                "eager_ms_per_step": round(e_ms, 4), "speedup": round(e_ms / ms, 3)}
    kt = r.kernel_times(steps)
    res = {"workload": DESCR[name], "ms_per_step": round(ms, 4),
           "kernels_us": {k: stats(v, 1e3) for k, v in kt.items() if v}}
    if r.work["kv_bytes"]:
        dms = mean_ms(kt["decode"])
        res["decode_kernel_us"] = round(dms * 1e3, 2)
        res["decode_kv_GBps_per_kernel"] = round(r.work["decode_bytes"] / (dms * 1e-3) / 1e9, 1)
        res["decode_frac_hbm_peak"] = round(res["decode_kv_GBps_per_kernel"] / HBM_PEAK_GBS, 4)
        if kt["merge"]:
            res["merge_kernel_us"] = round(mean_ms(kt["merge"]) * 1e3, 2)
        res["kv_GBps_per_step"] = round(r.work["kv_bytes"] / (ms * 1e-3) / 1e9, 1)
    if r.dense:
        res["gather_fresh_us"] = round(mean_ms(kt["append"]) * 1e3, 2)
        res["gather_with_prefix_us"] = r.gather_prefix_us()
    if r.work["prefill_flops"] and kt["prefill"]:
        pms = mean_ms(kt["prefill"])
        res["prefill_kernel_us"] = round(pms * 1e3, 2)
        res["prefill_TFLOPs_per_kernel"] = round(r.work["prefill_flops"] / (pms * 1e-3) / 1e12, 1)
        res["prefill_frac_mfma_peak"] = round(res["prefill_TFLOPs_per_kernel"] / MFMA_BF16_PEAK_TFS, 4)
        res["roofline"] = prefill_roofline(kt, r.work["prefill_flops"], name)
    elif r.work["prefill_flops"]:  # a mixed plan's one launch, timed as "decode"
        fms = mean_ms(kt["decode"])
        res["fused_decode_prefill_launch"] = True
        res["prefill_TFLOPs_in_fused_launch"] = round(r.work["prefill_flops"] / (fms * 1e-3) / 1e12, 1)
    if not r.dense:
        aux = aux_block(kt, aux_bytes(r.plan, r.w, r.append), name)
        if aux:
            res["aux_kernels"] = aux
    if with_cpu and name in CPU_BUDGET_S:
        res["cpu_baseline"] = cpu_baseline(r, CPU_BUDGET_S[name])
    del r
    import torch
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gqa_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured copy / bf16 GEMM ceilings")
    ap.add_argument("--waves-per-cu", type=int, default=0,
                    help="split-KV planner knob: decode waves per CU (0 = library default)")
    ap.add_argument("--min-chunk-pages", type=int, default=0,
                    help="split-KV planner knob (0 = library default)")
    ap.add_argument("--record-traffic", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL", "WORKLOAD", "COMMAND"),
                    help="write the traffic record of a kernel from two rocprofv3 --pmc csv files")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU code; rows, KV "
              "heads or a long row's pages would be split across GPUs, each running this "
              "kernel on its share.", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_attention_plan_amd import pkv  # noqa: F401  (fails loudly if not built)
    dev = torch.device("cuda:0")

    r = Runner(args.config, dev, args.waves_per_cu, args.min_chunk_pages)
    ms, wall_ms = r.time_steps(args.steps, args.warmup)
    kt = r.kernel_times(args.steps)
    w = r.work
    if r.graph:  # a replayed graph records no per-kernel events: whole steps only
        value, unit = w["kv_bytes"] / (ms * 1e-3) / 1e9, "GB/s"
        roof = None
    elif w["kv_bytes"]:  # decode rows present: KV bytes per second, decode kernel on HBM
        value, unit = w["kv_bytes"] / (ms * 1e-3) / 1e9, "GB/s"
        dec_ms = mean_ms(kt["decode"])
        achieved = w["decode_bytes"] / (dec_ms * 1e-3) / 1e9
        # a mixed plan runs decode and prefill in one launch (mixed_kernel)
        kname = "mixed_kernel" if w["prefill_flops"] and not kt["prefill"] else "decode_kernel"
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_of(kname, args.config) if kname in KERNEL_SOURCE else None,
                "kernel": kname, "kernel_us": round(dec_ms * 1e3, 2),
                "bytes_per_launch": w["decode_bytes"]}
    else:  # prefill only: FLOP per second, prefill kernel on bf16 MFMA
        value, unit = w["prefill_flops"] / (ms * 1e-3) / 1e12, "TFLOP/s"
        roof = prefill_roofline(kt, w["prefill_flops"], args.config)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCR[args.config], "kv_bytes_per_step": w["kv_bytes"],
                   "prefill_flops_per_step": w["prefill_flops"],
                   "step": r.step_descr},
        "roofline": roof,
        "kernels_us": {k: (round(mean_ms(v) * 1e3, 2) if v else None) for k, v in kt.items()},
        "kernels_us_dist": {k: stats(v, 1e3) for k, v in kt.items() if v},
        "host_ms_per_step": round(wall_ms, 4),
        "host": r.host_times(args.steps),
        "plan": r.plan.info(),
    }
    if not r.dense and not r.graph:
        aux = aux_block(kt, aux_bytes(r.plan, r.w, r.append), args.config)
        if aux:
            line["aux_kernels"] = aux
    per_cfg = {}
    if not args.no_cpu_baseline and args.config in CPU_BUDGET_S:
        per_cfg[args.config] = cpu_baseline(r, CPU_BUDGET_S[args.config])
        line["cpu_baseline"] = headline_cpu_baseline(per_cfg[args.config], unit, args.config)
    del r
    torch.cuda.empty_cache()
    if not args.no_secondary:
        sec = []
        for name in ("tiny_decode", "long_decode", "ragged_prefill", "mixed_window",
                     "gqa_decode_context_only", "ragged_prefill_dense", "tiny_decode_graph"):
            if name != args.config:
                res = secondary(name, dev, max(20, args.steps // 2), 5,
                                with_cpu=not args.no_cpu_baseline)
                if "cpu_baseline" in res:
                    per_cfg[name] = res.pop("cpu_baseline")
                if name == "ragged_prefill" and "roofline" in res:
                    line["roofline_prefill"] = res["roofline"]
                sec.append(res)
        line["secondary"] = sec
    if per_cfg:
        line["cpu_baseline_per_config"] = per_cfg
    if not args.no_ceilings:
        line["measured_ceilings"] = ceilings(dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
