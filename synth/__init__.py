"""Seeded synthetic workloads for batched attention over a paged KV cache.

This module builds inputs only: request lengths, the page table in CSR form,
query tensors and KV-cache pool contents.  It holds none of the attention
arithmetic; the oracle (oracle/) and the HIP path consume the bytes it makes.

Cache layout (mstar.engine.resources.attn.wrappers, module docstring and
FlashInferDecodeWrapper.run): one layer slice is
    [max_pages, 2, page_size, num_kv_heads, head_dim]
with index 0 of the "2" axis holding K and index 1 holding V.

CSR arrays (mstar.engine.resources.kv.plan, PagedIndptrs):
    qo_indptr[B+1], paged_kv_indptr[B+1], paged_kv_indices[nnz],
    paged_kv_last_page_len[B]   (all int32).
A row of kv_len N occupies ceil(N/page_size) pages; its last page holds
((N-1) % page_size) + 1 tokens (the rule the tiny-decode workload states).

Draw order for a seed: lengths, page permutation, q, pool contents, new K/V.
Integers come from numpy's PCG64 (default_rng(seed)); normals come from a
torch generator seeded with the same value on the device that holds the data,
float32 N(0,1) rounded to bfloat16.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "make_workload", "CONFIG_NAMES", "random_case", "from_lengths"]

# Short names for the five workloads this library is measured on.
CONFIG_NAMES = ("tiny_decode", "gqa_decode", "long_decode", "ragged_prefill", "mixed_window")


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                  # "decode" | "prefill" | "mixed"
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    causal: bool
    window_left: int
    max_pages: int
    kv_len: np.ndarray         # [B] int64, tokens in the cache per row (incl. this step's)
    q_len: np.ndarray          # [B] int64, query tokens per row
    qo_indptr: np.ndarray      # [B+1] int32
    kv_indptr: np.ndarray      # [B+1] int32
    kv_indices: np.ndarray     # [nnz] int32
    last_page_len: np.ndarray  # [B] int32
    q: torch.Tensor            # [T, Hq, D] bf16
    cache: torch.Tensor        # [max_pages, 2, ps, Hk, D] bf16
    k_new: Optional[torch.Tensor] = None   # [T, Hk, D] bf16 (tokens appended this step)
    v_new: Optional[torch.Tensor] = None
    max_prefill_rows: int = 0
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    def row_pages(self, r: int) -> np.ndarray:
        return self.kv_indices[self.kv_indptr[r]:self.kv_indptr[r + 1]]

    def to(self, device) -> "Workload":
        w = dataclasses.replace(self)
        w.q = self.q.to(device)
        w.cache = self.cache.to(device)
        if self.k_new is not None:
            w.k_new = self.k_new.to(device)
            w.v_new = self.v_new.to(device)
        return w


def _normals(gen: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)


def from_lengths(name, kind, kv_len, q_len, *, num_qo_heads, num_kv_heads, head_dim, page_size,
                 causal=True, window_left=-1, pool_pages=None, rng=None, seed=0, device="cpu",
                 stale="zero", new_tokens=False, max_prefill_rows=0, gen=None,
                 page_order="random", layout_only=False) -> Workload:
    """Lay rows of the given lengths out in a page pool and fill it.

    kv_len counts every token of the row, including the ones queried this step
    (those sit at the end: [cached prefix | fresh tokens]).  stale="zero"|"nan"
    selects what unused pages and slots past the last token hold.
    page_order: "random" (seeded permutation of the pool) or "sequential".
    layout_only: the page table and lengths only (q, cache empty), e.g. for
    planner checks at full size; the page ids are those of the full workload.
    """
    kv_len = np.asarray(kv_len, dtype=np.int64)
    q_len = np.asarray(q_len, dtype=np.int64)
    assert kv_len.shape == q_len.shape
    assert np.all(q_len <= kv_len) and np.all(kv_len >= 1)
    rng = rng if rng is not None else np.random.default_rng(seed)
    ps = page_size
    npages = (kv_len + ps - 1) // ps
    nnz = int(npages.sum())
    pool = int(pool_pages) if pool_pages is not None else max(nnz, 1)
    assert pool >= nnz, "pool too small"
    if page_order == "random":
        ids = rng.permutation(pool)[:nnz].astype(np.int32)
    else:
        ids = np.arange(nnz, dtype=np.int32)
    kv_indptr = np.zeros(kv_len.shape[0] + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(npages)
    qo_indptr = np.zeros(kv_len.shape[0] + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(q_len)
    last_page_len = (((kv_len - 1) % ps) + 1).astype(np.int32)

    if layout_only:
        empty = torch.empty(0, dtype=torch.bfloat16)
        return Workload(name=name, kind=kind, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, page_size=ps, causal=causal, window_left=window_left,
                        max_pages=pool, kv_len=kv_len, q_len=q_len, qo_indptr=qo_indptr,
                        kv_indptr=kv_indptr, kv_indices=ids, last_page_len=last_page_len,
                        q=empty, cache=empty, max_prefill_rows=max_prefill_rows, seed=seed)
    gen = gen if gen is not None else torch.Generator(device=device).manual_seed(seed)
    T = int(qo_indptr[-1])
    q = _normals(gen, (T, num_qo_heads, head_dim), device)

    fill = float("nan") if stale == "nan" else 0.0
    cache = torch.full((pool, 2, ps, num_kv_heads, head_dim), fill, dtype=torch.bfloat16, device=device)
    # Used pages get N(0,1) contents, written in chunks to bound temporary memory.
    ids_t = torch.from_numpy(ids.astype(np.int64)).to(device)
    chunk = max(1, (1 << 27) // (2 * ps * num_kv_heads * head_dim))
    for s in range(0, nnz, chunk):
        e = min(nnz, s + chunk)
        vals = _normals(gen, (e - s, 2, ps, num_kv_heads, head_dim), device)
        cache.index_copy_(0, ids_t[s:e], vals)
    # Slots past the last token of each row's last page are stale.
    if nnz:
        last_ids = ids[kv_indptr[1:] - 1]
        for r in np.nonzero(last_page_len < ps)[0]:
            cache[int(last_ids[r]), :, int(last_page_len[r]):] = fill

    k_new = v_new = None
    if new_tokens:
        k_new = _normals(gen, (T, num_kv_heads, head_dim), device)
        v_new = _normals(gen, (T, num_kv_heads, head_dim), device)

    return Workload(name=name, kind=kind, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, page_size=ps, causal=causal, window_left=window_left,
                    max_pages=pool, kv_len=kv_len, q_len=q_len, qo_indptr=qo_indptr,
                    kv_indptr=kv_indptr, kv_indices=ids, last_page_len=last_page_len, q=q,
                    cache=cache, k_new=k_new, v_new=v_new, max_prefill_rows=max_prefill_rows,
                    seed=seed)


def make_workload(name: str, *, seed: Optional[int] = None, device="cpu", stale="zero",
                  scale_rows: Optional[int] = None, layout_only: bool = False) -> Workload:
    """One of the five named workloads.

    Default seed is 1000 + (1-based position in CONFIG_NAMES).  scale_rows, when
    given, keeps only that many rows (a cut-down sample with the same
    distributions, used where the full size does not fit a CPU test).
    """
    k = CONFIG_NAMES.index(name) + 1
    seed = 1000 + k if seed is None else seed
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device).manual_seed(seed)
    common = dict(rng=rng, seed=seed, device=device, stale=stale, gen=gen, layout_only=layout_only)

    def cut(*arrs):
        if scale_rows is None:
            return arrs
        return tuple(a[:scale_rows] for a in arrs)

    if name == "tiny_decode":
        B = 4
        kv = rng.integers(1, 101, size=B)
        (kv,) = cut(kv)
        return from_lengths(name, "decode", kv, np.ones_like(kv), num_qo_heads=4, num_kv_heads=2,
                            head_dim=64, page_size=16, pool_pages=32, new_tokens=False, **common)
    if name == "gqa_decode":
        B = 128
        kv = rng.integers(512, 4097, size=B)
        (kv,) = cut(kv)
        return from_lengths(name, "decode", kv, np.ones_like(kv), num_qo_heads=32, num_kv_heads=8,
                            head_dim=128, page_size=16, pool_pages=40000, new_tokens=True, **common)
    if name == "long_decode":
        B = 8
        kv = rng.integers(32768, 131073, size=B)
        (kv,) = cut(kv)
        return from_lengths(name, "decode", kv, np.ones_like(kv), num_qo_heads=32, num_kv_heads=8,
                            head_dim=128, page_size=16, pool_pages=None, **common)
    if name == "ragged_prefill":
        B = 16
        ql = rng.integers(128, 2049, size=B)
        prefix = rng.integers(0, 4097, size=B)
        ql, prefix = cut(ql, prefix)
        return from_lengths(name, "prefill", prefix + ql, ql, num_qo_heads=32, num_kv_heads=8,
                            head_dim=128, page_size=16, causal=True, pool_pages=None, **common)
    if name == "mixed_window":
        n_dec, n_pre = 256, 4
        dec_kv = rng.integers(256, 8193, size=n_dec)
        kv = np.concatenate([dec_kv, np.full(n_pre, 2048 + 1024)])
        ql = np.concatenate([np.ones(n_dec, dtype=np.int64), np.full(n_pre, 1024)])
        order = rng.permutation(n_dec + n_pre)
        kv, ql = kv[order], ql[order]
        if scale_rows is not None:
            # keep every prompt row plus the first decode rows
            keep = np.concatenate([np.nonzero(ql > 1)[0], np.nonzero(ql == 1)[0][:scale_rows]])
            keep.sort()
            kv, ql = kv[keep], ql[keep]
        return from_lengths(name, "mixed", kv, ql, num_qo_heads=16, num_kv_heads=16, head_dim=64,
                            page_size=32, causal=True, window_left=4096, pool_pages=None,
                            max_prefill_rows=n_pre, **common)
    raise KeyError(name)


def random_case(seed: int, *, batch=3, num_qo_heads=4, num_kv_heads=2, head_dim=16, page_size=4,
                max_kv=40, kind="prefill", causal=True, window_left=-1, device="cpu",
                stale="zero", extra_pages=5, new_tokens=False) -> Workload:
    """A small random case for brute-force checks.  Rows may have q_len 0."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(1, max_kv + 1, size=batch)
    if kind == "decode":
        ql = np.ones_like(kv)
    else:
        ql = np.array([rng.integers(0, k + 1) for k in kv], dtype=np.int64)
    npages = int(((kv + page_size - 1) // page_size).sum())
    return from_lengths(f"random{seed}", kind, kv, ql, num_qo_heads=num_qo_heads,
                        num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                        causal=causal, window_left=window_left, pool_pages=npages + extra_pages,
                        rng=rng, seed=seed, device=device, stale=stale, new_tokens=new_tokens)
