"""float64 reference for paged-KV attention, KV append and the mixed permutation.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain definitions, no
blocking, no fusion: a reader should be able to check each function against the
documentation pages by eye.

Conventions that no page fixes ("parity unpinned"):
  * on the "2" axis of a cache layer slice, index 0 is K and index 1 is V;
  * query head h reads KV head h // (num_qo_heads // num_kv_heads).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "bf16_to_f64", "RowLayout", "decode_csr", "query_position", "visible_keys",
    "kv_head_of", "gather_row_kv", "attention", "attention_rows", "attention_bruteforce", "write_slots",
    "apply_append", "mixed_permutation", "merge_partials", "context_only_views",
    "attention_dense", "dense_gather", "OracleError",
]


class OracleError(ValueError):
    """Raised for inputs that violate the page-table definition."""


def bf16_to_f64(x) -> np.ndarray:
    """bfloat16 values to float64, exactly.

    Accepts a torch bf16 tensor (any device), a numpy uint16 array of bf16 bit
    patterns, or any numpy float array (converted with astype).  A bf16 value is
    the upper 16 bits of an IEEE binary32, so widening is exact.
    """
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch
        bits = x.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    else:
        bits = np.asarray(x)
        if bits.dtype != np.uint16:
            return bits.astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class RowLayout:
    """What the page table says about one request row."""
    pages: np.ndarray   # physical page ids in logical order
    kv_len: int         # tokens in the cache for this row (this step's included)
    q_len: int          # query tokens this step


def decode_csr(page_size, kv_indptr, kv_indices, last_page_len, *, max_pages, qo_indptr=None,
               kv_lens=None) -> list[RowLayout]:
    """Decode the CSR page table into per-row layouts and validate it.

    A row owns pages kv_indices[kv_indptr[r]:kv_indptr[r+1]] (kv.plan,
    PagedIndptrs).  Its last page holds last_page_len[r] tokens, between 1 and
    page_size, and every earlier page is full, so
        kv_len = (num_pages - 1) * page_size + last_page_len
    (kv.plan, SequenceView.last_page_len).  Query rows come from qo_indptr
    (absent for decode: one query per row).  A row's query tokens are the last
    q_len tokens of its KV, so q_len <= kv_len.
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    last_page_len = np.asarray(last_page_len, dtype=np.int64)
    B = len(last_page_len)
    if kv_indptr.shape != (B + 1,) or kv_indptr[0] != 0:
        raise OracleError("paged_kv_indptr must have batch+1 entries starting at 0")
    if qo_indptr is None:
        qo_indptr = np.arange(B + 1, dtype=np.int64)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    if qo_indptr.shape != (B + 1,) or qo_indptr[0] != 0:
        raise OracleError("qo_indptr must have batch+1 entries starting at 0")
    rows = []
    for r in range(B):
        n_pages = kv_indptr[r + 1] - kv_indptr[r]
        if n_pages < 1:
            raise OracleError(f"row {r}: no pages")
        if kv_indptr[r + 1] > len(kv_indices):
            raise OracleError(f"row {r}: indptr past the index array")
        lpl = last_page_len[r]
        if not (1 <= lpl <= page_size):
            raise OracleError(f"row {r}: last_page_len {lpl} outside [1, {page_size}]")
        pages = kv_indices[kv_indptr[r]:kv_indptr[r + 1]]
        if np.any(pages < 0) or np.any(pages >= max_pages):
            raise OracleError(f"row {r}: page id outside [0, {max_pages})")
        kv_len = int((n_pages - 1) * page_size + lpl)
        q_len = int(qo_indptr[r + 1] - qo_indptr[r])
        if q_len < 0 or q_len > kv_len:
            raise OracleError(f"row {r}: q_len {q_len} not in [0, kv_len={kv_len}]")
        if kv_lens is not None and int(kv_lens[r]) != kv_len:
            raise OracleError(f"row {r}: kv_lens {kv_lens[r]} != {kv_len}")
        rows.append(RowLayout(pages=pages, kv_len=kv_len, q_len=q_len))
    return rows


def query_position(kv_len: int, q_len: int, t: int) -> int:
    """Sequence position of query token t of a row: the queries are the last
    q_len tokens of the row's [cached prefix | fresh tokens] sequence."""
    return kv_len - q_len + t


def visible_keys(p: int, kv_len: int, causal: bool, window_left: int) -> tuple[int, int]:
    """Inclusive key range [lo, hi] a query at position p attends to.

    Causal: keys up to and including p.  window_left w >= 0: the query sees the
    w positions before it and itself, so keys >= p - w; -1 means no bound
    (FlashInferPrefillWrapper.plan; the decode plan uses the same rule).
    """
    hi = p if causal else kv_len - 1
    lo = 0 if window_left < 0 else max(0, p - window_left)
    return lo, hi


def kv_head_of(h: int, num_qo_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: consecutive query heads share a KV head
    (group = num_qo_heads // num_kv_heads).  A convention; parity unpinned."""
    return h // (num_qo_heads // num_kv_heads)


def gather_row_kv(cache, pages, kv_len: int, page_size: int):
    """Logical K and V of one row, [kv_len, num_kv_heads, head_dim] float64 each.

    Token j of the row lives on page pages[j // page_size], slot j % page_size;
    cache axis 1 index 0 is K and index 1 is V (layer slice layout
    [max_pages, 2, page_size, num_kv_heads, head_dim]).
    """
    c = cache if isinstance(cache, np.ndarray) and cache.dtype == np.float64 else None
    n_pages = (kv_len + page_size - 1) // page_size
    parts = []
    for i in range(n_pages):
        blk = cache[int(pages[i])]
        parts.append(blk if c is not None else bf16_to_f64(blk))
    allp = np.stack(parts)  # [n_pages, 2, ps, Hk, D]
    K = allp[:, 0].reshape(n_pages * page_size, *allp.shape[3:])[:kv_len]
    V = allp[:, 1].reshape(n_pages * page_size, *allp.shape[3:])[:kv_len]
    return K, V


def _attend_head(qh, K, V, pos, kv_len, causal, window_left, scale):
    """Queries of one head over one row.

    qh [n, D] float64 at sequence positions pos [n]; K, V [kv_len, D].
    s_tj = scale * q_t . k_j over the visible keys (visible_keys), then
    o_t = sum_j softmax(s_t)_j v_j and lse_t = ln sum_j exp(s_tj).
    """
    s = scale * (qh @ K.T)                                   # [n, kv_len]
    j = np.arange(kv_len)[None, :]
    lo = np.array([visible_keys(int(p), kv_len, causal, window_left)[0] for p in pos])[:, None]
    hi = np.array([visible_keys(int(p), kv_len, causal, window_left)[1] for p in pos])[:, None]
    s = np.where((j >= lo) & (j <= hi), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    denom = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(denom))[:, 0]
    o = (e / denom) @ V
    return o, lse


def attention_rows(q, cache, page_size, kv_indptr, kv_indices, last_page_len, *, num_qo_heads,
                   num_kv_heads, qo_indptr=None, causal=True, window_left=-1, rows=None,
                   max_pages=None, tokens=None):
    """Reference attention for selected rows.

    Returns {r: (out [n, Hq, D] float64, lse [n, Hq] float64)} where n is the
    row's q_len, or len(tokens[r]) when tokens = {r: [token indices]} picks a
    subset.  q is [total_q, Hq, D]; cache is the layer slice.  The scale is
    1/sqrt(head_dim); lse is the natural log-sum-exp of the scaled logits.
    """
    max_pages = cache.shape[0] if max_pages is None else max_pages
    layout = decode_csr(page_size, kv_indptr, kv_indices, last_page_len, max_pages=max_pages,
                        qo_indptr=qo_indptr)
    if qo_indptr is None:
        qo_indptr = np.arange(len(layout) + 1)
    if num_qo_heads % num_kv_heads:
        raise OracleError("num_qo_heads must be a multiple of num_kv_heads")
    group = num_qo_heads // num_kv_heads
    rows = range(len(layout)) if rows is None else rows
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D)
    res = {}
    for r in rows:
        lay = layout[r]
        toks = np.arange(lay.q_len) if tokens is None else np.asarray(tokens[r], dtype=np.int64)
        q0 = int(qo_indptr[r])
        qr = bf16_to_f64(q[q0:q0 + lay.q_len])[toks] if lay.q_len else np.zeros((0, num_qo_heads, D))
        pos = np.array([query_position(lay.kv_len, lay.q_len, int(t)) for t in toks], dtype=np.int64)
        out = np.zeros((len(toks), num_qo_heads, D))
        lse = np.zeros((len(toks), num_qo_heads))
        if len(toks):
            K, V = gather_row_kv(cache, lay.pages, lay.kv_len, page_size)
            for h in range(num_qo_heads):
                hk = kv_head_of(h, num_qo_heads, num_kv_heads)
                out[:, h], lse[:, h] = _attend_head(qr[:, h], K[:, hk], V[:, hk], pos, lay.kv_len,
                                                    causal, window_left, scale)
        res[r] = (out, lse)
    return res


def attention(q, cache, page_size, kv_indptr, kv_indices, last_page_len, *, num_qo_heads,
              num_kv_heads, qo_indptr=None, causal=True, window_left=-1, max_pages=None):
    """Reference attention for every row, packed like q: (out [T,Hq,D], lse [T,Hq])."""
    res = attention_rows(q, cache, page_size, kv_indptr, kv_indices, last_page_len,
                         num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                         qo_indptr=qo_indptr, causal=causal, window_left=window_left,
                         max_pages=max_pages)
    T = q.shape[0]
    out = np.zeros((T, num_qo_heads, q.shape[-1]))
    lse = np.zeros((T, num_qo_heads))
    qo = np.arange(len(res) + 1) if qo_indptr is None else np.asarray(qo_indptr)
    for r, (o, l) in res.items():
        out[qo[r]:qo[r + 1]] = o
        lse[qo[r]:qo[r + 1]] = l
    return out, lse


def attention_dense(q, k, v, cu_q, cu_k, *, num_qo_heads, num_kv_heads, causal=True,
                    window_left=-1):
    """Attention over contiguous [frozen prefix | fresh tokens] K/V
    (attn.dense, DenseAttentionManager and DensePlan): row r's queries are
    q[cu_q[r]:cu_q[r+1]] and its keys k/v[cu_k[r]:cu_k[r+1]], the last q_len of
    them fresh, so query t sits at position kv_len - q_len + t exactly as for a
    paged row.  q [Tq, Hq, D], k/v [Tk, Hk, D] (bf16 bits or float64).
    Returns (out [Tq, Hq, D], lse [Tq, Hq]) float64."""
    cq = np.asarray(cu_q, dtype=np.int64)
    ck = np.asarray(cu_k, dtype=np.int64)
    Q, K, V = bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v)
    D = Q.shape[-1]
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((Q.shape[0], num_qo_heads, D))
    lse = np.zeros((Q.shape[0], num_qo_heads))
    for r in range(len(cq) - 1):
        L, n = int(cq[r + 1] - cq[r]), int(ck[r + 1] - ck[r])
        if L > n:
            raise OracleError(f"row {r}: q_len {L} > kv_len {n}")
        if L == 0:
            continue
        pos = np.array([query_position(n, L, t) for t in range(L)], dtype=np.int64)
        for h in range(num_qo_heads):
            hk = kv_head_of(h, num_qo_heads, num_kv_heads)
            o, l = _attend_head(Q[cq[r]:cq[r + 1], h], K[ck[r]:ck[r + 1], hk],
                                V[ck[r]:ck[r + 1], hk], pos, n, causal, window_left, scale)
            out[cq[r]:cq[r + 1], h], lse[cq[r]:cq[r + 1], h] = o, l
    return out, lse


def dense_gather(cache_bits, page_size, kv_indptr, kv_indices, cu_q, cu_k, k_fresh_bits,
                 v_fresh_bits, *, with_prefix=True, k_out=None, v_out=None):
    """Contiguous K/V of a dense plan (DenseAttentionManager: the prefix is
    gathered from the pages, the step's fresh K/V concatenated after it).
    Row r's prefix is its first (cu_k[r+1]-cu_k[r]) - (cu_q[r+1]-cu_q[r]) tokens,
    token j on page kv_indices[kv_indptr[r] + j // page_size] at slot
    j % page_size; its fresh tokens are k/v_fresh[cu_q[r]:cu_q[r+1]].  Bit
    copies (uint16).  with_prefix=False leaves the prefix rows of k_out/v_out as
    given.  Returns (k_out, v_out) [cu_k[-1], Hk, D]."""
    cq = np.asarray(cu_q, dtype=np.int64)
    ck = np.asarray(cu_k, dtype=np.int64)
    shape = (int(ck[-1]),) + tuple(k_fresh_bits.shape[1:])
    ko = np.zeros(shape, np.uint16) if k_out is None else k_out.copy()
    vo = np.zeros(shape, np.uint16) if v_out is None else v_out.copy()
    for r in range(len(cq) - 1):
        L, n = int(cq[r + 1] - cq[r]), int(ck[r + 1] - ck[r])
        P = n - L
        if with_prefix:
            for j in range(P):
                page = int(kv_indices[int(kv_indptr[r]) + j // page_size])
                ko[ck[r] + j] = cache_bits[page, 0, j % page_size]
                vo[ck[r] + j] = cache_bits[page, 1, j % page_size]
        ko[ck[r] + P:ck[r + 1]] = k_fresh_bits[cq[r]:cq[r + 1]]
        vo[ck[r] + P:ck[r + 1]] = v_fresh_bits[cq[r]:cq[r + 1]]
    return ko, vo


def attention_bruteforce(q, cache, page_size, kv_indptr, kv_indices, last_page_len, *,
                         num_qo_heads, num_kv_heads, qo_indptr=None, causal=True, window_left=-1):
    """Scalar-loop attention for tiny inputs: walks every (token, head, key)
    with Python floats and math.exp; no numpy reductions, no gather helper.

    Key j of a row is read at cache[page, 0|1, slot] where the page is found by
    counting page_size tokens per page through the row's page list.
    """
    Q = bf16_to_f64(q)
    C = bf16_to_f64(cache)
    B = len(last_page_len)
    qo = list(range(B + 1)) if qo_indptr is None else [int(x) for x in qo_indptr]
    D = Q.shape[-1]
    group = num_qo_heads // num_kv_heads
    T = Q.shape[0]
    out = [[[0.0] * D for _ in range(num_qo_heads)] for _ in range(T)]
    lse = [[0.0] * num_qo_heads for _ in range(T)]
    for r in range(B):
        pages = [int(x) for x in kv_indices[int(kv_indptr[r]):int(kv_indptr[r + 1])]]
        kv_len = 0
        slots = []          # (page, slot) of each logical token, in order
        for i, pg in enumerate(pages):
            fill = page_size if i < len(pages) - 1 else int(last_page_len[r])
            for s in range(fill):
                slots.append((pg, s))
                kv_len += 1
        L = qo[r + 1] - qo[r]
        for t in range(L):
            pos = kv_len - L + t
            for h in range(num_qo_heads):
                hk = h // group
                logits = []
                for j in range(kv_len):
                    if causal and j > pos:
                        continue
                    if window_left >= 0 and j < pos - window_left:
                        continue
                    pg, s = slots[j]
                    acc = 0.0
                    for d in range(D):
                        acc += Q[qo[r] + t, h, d] * C[pg, 0, s, hk, d]
                    logits.append((j, acc / math.sqrt(D)))
                mx = max(v for _, v in logits)
                tot = sum(math.exp(v - mx) for _, v in logits)
                for d in range(D):
                    acc = 0.0
                    for j, v in logits:
                        pg, s = slots[j]
                        acc += math.exp(v - mx) / tot * C[pg, 1, s, hk, d]
                    out[qo[r] + t][h][d] = acc
                lse[qo[r] + t][h] = mx + math.log(tot)
    return np.array(out).reshape(T, num_qo_heads, D), np.array(lse).reshape(T, num_qo_heads)


def write_slots(page_size, kv_indptr, kv_indices, last_page_len, *, qo_indptr=None):
    """Flat cache slot (page * page_size + offset) of every query token.

    Token t of row r sits at position p = kv_len - q_len + t, so it is stored on
    page kv_indices[kv_indptr[r] + p // page_size] at offset p % page_size.  For
    decode (one token per row) that is the row's last page at offset
    last_page_len - 1: the page table handed to the plan already counts the new
    token (FlashInferDecodeWrapper.plan; kv.plan KVPlanOutput decode_pages /
    decode_offsets).  Returns int64 [total_q].
    """
    B = len(last_page_len)
    qo = np.arange(B + 1) if qo_indptr is None else np.asarray(qo_indptr, dtype=np.int64)
    out = np.zeros(int(qo[-1]), dtype=np.int64)
    for r in range(B):
        n_pages = int(kv_indptr[r + 1] - kv_indptr[r])
        kv_len = (n_pages - 1) * page_size + int(last_page_len[r])
        L = int(qo[r + 1] - qo[r])
        for t in range(L):
            p = kv_len - L + t
            page = int(kv_indices[int(kv_indptr[r]) + p // page_size])
            out[qo[r] + t] = page * page_size + p % page_size
    return out


def apply_append(cache_bits: np.ndarray, slots, k_new_bits: np.ndarray, v_new_bits: np.ndarray,
                 page_size: int) -> np.ndarray:
    """Cache after storing each new token's K and V at its slot (bit copy).

    cache_bits: uint16 [max_pages, 2, ps, Hk, D]; k/v_new_bits: uint16 [T, Hk, D].
    """
    out = cache_bits.copy()
    for t, flat in enumerate(np.asarray(slots)):
        page, off = int(flat) // page_size, int(flat) % page_size
        out[page, 0, off] = k_new_bits[t]
        out[page, 1, off] = v_new_bits[t]
    return out


def context_only_views(page_size, kv_indptr, kv_indices, last_page_len, to_compute, query_spans):
    """The page table of a step's rows without the tokens the step appends
    (kv.plan, context_only_views): row r keeps its first
    kv_len - to_compute[r] tokens, the pages past them are dropped, and its
    query count becomes query_spans[r].  Every row must keep at least one
    stored token (0 <= to_compute < kv_len) and query_spans[r] >= 0.
    Returns (kv_indptr, kv_indices, last_page_len, qo_indptr) of the new views.
    """
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    indices = np.asarray(kv_indices, dtype=np.int64)
    lpl = np.asarray(last_page_len, dtype=np.int64)
    B = len(lpl)
    new_ptr, new_idx, new_lpl, qo = [0], [], [], [0]
    for r in range(B):
        pages = indices[indptr[r]:indptr[r + 1]]
        if len(pages) < 1 or not (1 <= lpl[r] <= page_size):
            raise OracleError(f"row {r}: malformed page table")
        kv_len = (len(pages) - 1) * page_size + int(lpl[r])
        tc, qs = int(to_compute[r]), int(query_spans[r])
        if not (0 <= tc < kv_len):
            raise OracleError(f"row {r}: to_compute {tc} must lie in [0, kv_len={kv_len})")
        if qs < 0:
            raise OracleError(f"row {r}: query_spans {qs} < 0")
        kept = kv_len - tc
        n_pages = -(-kept // page_size)
        new_idx.extend(int(p) for p in pages[:n_pages])
        new_ptr.append(new_ptr[-1] + n_pages)
        new_lpl.append(kept - (n_pages - 1) * page_size)
        qo.append(qo[-1] + qs)
    as32 = lambda a: np.asarray(a, dtype=np.int32)
    return as32(new_ptr), as32(new_idx), as32(new_lpl), as32(qo)


def mixed_permutation(qo_indptr, *, max_prefill_rows):
    """Split a mixed step's rows and order the prompt tokens first.

    Rows with exactly one query token go to the decode plan; rows with two or
    more are prompt rows for the prefill plan, at most max_prefill_rows of them
    (FlashInferMixedWrapper).  perm lists, row by row in ascending order, the
    packed-q indices of every prompt token: prefill position i reads q[perm[i]]
    and writes out[perm[i]].  Rows with no query tokens are in neither plan.
    Returns (decode_rows, prompt_rows, perm).
    """
    qo = np.asarray(qo_indptr, dtype=np.int64)
    lens = qo[1:] - qo[:-1]
    decode_rows = np.nonzero(lens == 1)[0].astype(np.int32)
    prompt_rows = np.nonzero(lens >= 2)[0].astype(np.int32)
    if len(prompt_rows) > max_prefill_rows:
        raise OracleError(f"{len(prompt_rows)} prompt rows > max_prefill_rows={max_prefill_rows}")
    perm = [np.arange(qo[r], qo[r + 1]) for r in prompt_rows]
    perm = np.concatenate(perm).astype(np.int32) if perm else np.zeros(0, dtype=np.int32)
    return decode_rows, prompt_rows, perm


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine attention over disjoint key chunks.

    Given, per chunk c, o_c (softmax-weighted V over that chunk alone) and lse_c,
    the result over the union is lse = ln sum_c exp(lse_c) and
    o = sum_c exp(lse_c - lse) o_c (split-KV partials,
    mstar.engine.resources.attn.workspace).  o_parts [C, ..., D], lse_parts [C, ...].
    """
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m)
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    o = (w[..., None] * o_parts).sum(axis=0) / tot[..., None]
    return o, lse
