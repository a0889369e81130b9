"""Checks for the planner's integer output.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Two kinds of check:
  * cover checks, which hold for any valid plan: decode tiles cover every
    visible key of every (row, KV head) exactly once; prefill tiles cover every
    (row, KV head, query token) exactly once with a key range containing that
    token's visible keys; split-KV partial slots are unique and merged once;
  * a restatement of the documented tiling policy in plain Python (the pages
    say only that a plan's size depends on rows, heads and the CU count,
    mstar.engine.resources.attn.workspace, Workspace), so the planner's tile
    lists can be compared bit for bit.

Policy (the same rules the header documents):
  decode rows   visible keys [lo, N-1]; pages fp = lo // ps .. lp = (N-1) // ps.
                W = max(1, num_cus * waves_per_cu // Hk) workers (waves_per_cu
                4 for group 1, 2, 4 and 16 for group 8 unless given).  Rows sorted by
                visible pages descending (ties: row index) are poured, in that
                order, into workers of capacity C: a piece of p pages costs
                p + 2; a worker takes min(remaining pages of the row, C - used -
                2) pages of the row when that is >= 1, else the next worker
                starts.  C is the smallest value >= max(min_chunk_pages,
                ceil(total / W)) + 2 (total = pages + 2 per row) whose pour
                needs at most W workers.  Per row pieces in order, per piece
                tiles head-minor.  Rows with more than one piece get
                Hk * n_pieces consecutive partial slots, head-major.
  prefill rows  blocks of 192 // group query tokens; per block keys
                [lo(first token), hi(last token)]; tiles sorted by key count
                descending, ties by (row, block, head).
"""
from __future__ import annotations

import numpy as np

from .reference import decode_csr, query_position, visible_keys

__all__ = ["decode_policy", "prefill_policy", "check_decode_cover", "check_prefill_cover",
           "split_rows"]


def split_rows(kind, layout, max_prefill_rows=0):
    """Which rows go to the decode plan and which to the prefill plan."""
    if kind == "decode":
        return [r for r in range(len(layout))], []
    if kind == "prefill":
        return [], [r for r, l in enumerate(layout) if l.q_len >= 1]
    dec = [r for r, l in enumerate(layout) if l.q_len == 1]
    pre = [r for r, l in enumerate(layout) if l.q_len >= 2]
    if len(pre) > max_prefill_rows:
        raise ValueError("more prompt rows than max_prefill_rows")
    return dec, pre


def _pour(pages, cap, cost=2):
    """Pieces (row position, first page offset, page count, worker) of pouring
    rows of `pages` pages, in order, into workers of capacity `cap`."""
    pieces, w, used = [], 0, 0
    for i, v in enumerate(pages):
        done = 0
        while done < v:
            if cap - used - cost < 1:
                w, used = w + 1, 0
            take = min(v - done, cap - used - cost)
            pieces.append((i, done, take, w))
            used += take + cost
            done += take
    return pieces


def decode_policy(layout, rows, *, page_size, num_kv_heads, window_left, num_cus, qo_indptr,
                  kv_indptr, group, waves_per_cu=0, min_chunk_pages=8):
    """Expected decode tiles, merges and worker table.

    Returns (tiles, merges, capacity, n_slots, work) with tiles as tuples
    (row, kv_head, kv_start, kv_end, page_base, q_index, out_slot, kv_len),
    merges as (q_index, kv_head, slot_base, n_chunks) and work the first piece
    of every used worker followed by the piece count.
    """
    ps, hk_n = page_size, num_kv_heads
    wpc = waves_per_cu or (16 if group == 8 else 4)
    W = max(1, num_cus * wpc // hk_n)
    info = {}
    for r in rows:
        n = layout[r].kv_len
        lo, _ = visible_keys(n - 1, n, True, window_left)
        fp, lp = lo // ps, (n - 1) // ps
        info[r] = (lo, fp, lp, lp - fp + 1)
    order = sorted(rows, key=lambda r: (-info[r][3], r))
    pages = [info[r][3] for r in order]
    total = sum(v + 2 for v in pages)
    cap = max(min_chunk_pages, -(-total // W)) + 2
    if pages:
        while _pour(pages, cap)[-1][3] + 1 > W:
            cap += 1
    pieces = _pour(pages, cap)
    n_pieces = [sum(1 for p in pieces if p[0] == i) for i in range(len(order))]
    base, slot, merges = {}, 0, []
    for i, r in enumerate(order):
        if n_pieces[i] > 1:
            base[i] = slot
            for hk in range(hk_n):
                merges.append((int(qo_indptr[r]), hk, slot + hk * n_pieces[i], n_pieces[i]))
            slot += hk_n * n_pieces[i]
    tiles, work, seen = [], [], {}
    for k, (i, off, take, w) in enumerate(pieces):
        while len(work) <= w:
            work.append(k)
        r = order[i]
        lo, fp, lp, vis = info[r]
        n = layout[r].kv_len
        c = seen.get(i, 0)
        seen[i] = c + 1
        ks = max(lo, (fp + off) * ps)
        ke = min(n, (fp + off + take) * ps)
        for hk in range(hk_n):
            out_slot = base[i] + hk * n_pieces[i] + c if i in base else -1
            tiles.append((r, hk, ks, ke, int(kv_indptr[r]), int(qo_indptr[r]), out_slot, n))
    work.append(len(pieces))
    return tiles, merges, cap, slot, work


# (query head, token) pairs of one prefill tile under the library's documented
# policy.
TILE_PAIRS = 192


def prefill_policy(layout, rows, *, num_qo_heads, num_kv_heads, causal, window_left, qo_indptr,
                   kv_indptr):
    """Expected prefill tiles as tuples
    (row, kv_head, q_start, q_count, kv_lo, kv_hi, page_base, q_base, kv_len, q_len)."""
    group = num_qo_heads // num_kv_heads
    bt = TILE_PAIRS // group
    items = []
    for r in rows:
        n, L = layout[r].kv_len, layout[r].q_len
        for b in range(-(-L // bt)):
            qs = b * bt
            qc = min(bt, L - qs)
            lo, _ = visible_keys(query_position(n, L, qs), n, causal, window_left)
            _, hi = visible_keys(query_position(n, L, qs + qc - 1), n, causal, window_left)
            for hk in range(num_kv_heads):
                items.append(((-(hi - lo + 1), r, b, hk),
                              (r, hk, qs, qc, lo, hi, int(kv_indptr[r]), int(qo_indptr[r]), n, L)))
    items.sort(key=lambda x: x[0])
    return [t for _, t in items]


def check_decode_cover(tiles, merges, layout, rows, *, num_kv_heads, window_left, n_slots):
    """Every visible key of every (decode row, KV head) in exactly one tile;
    partial slots unique, in range, and merged exactly once in chunk order."""
    seen = {}
    slots = set()
    for (r, hk, ks, ke, _pb, _qi, slot, _n) in tiles:
        assert 0 <= ks < ke, (r, hk, ks, ke)
        seen.setdefault((r, hk), []).append((ks, ke, slot))
        if slot >= 0:
            assert slot not in slots and slot < n_slots
            slots.add(slot)
    assert set(seen) == {(r, hk) for r in rows for hk in range(num_kv_heads)}
    merged = set()
    mslots = {}
    for (qi, hk, base, nch) in merges:
        assert nch > 1
        mslots[(qi, hk)] = list(range(base, base + nch))
        merged.update(range(base, base + nch))
    assert merged == slots
    for (r, hk), parts in seen.items():
        n = layout[r].kv_len
        lo, hi = visible_keys(n - 1, n, True, window_left)
        parts.sort()
        assert parts[0][0] == lo and parts[-1][1] == hi + 1
        for a, b in zip(parts, parts[1:]):
            assert a[1] == b[0]
        if len(parts) > 1:
            assert all(p[2] >= 0 for p in parts)
        else:
            assert parts[0][2] == -1


def check_prefill_cover(tiles, layout, rows, *, num_kv_heads, causal, window_left):
    """Every (prefill row, KV head, query token) in exactly one tile, whose key
    range contains that token's visible keys."""
    count = {}
    for (r, hk, qs, qc, klo, khi, _pb, _qb, n, L) in tiles:
        assert qc >= 1 and 0 <= qs and qs + qc <= L
        for t in range(qs, qs + qc):
            lo, hi = visible_keys(query_position(n, L, t), n, causal, window_left)
            assert klo <= lo and hi <= khi, (r, t, lo, hi, klo, khi)
            count[(r, hk, t)] = count.get((r, hk, t), 0) + 1
    want = {(r, hk, t) for r in rows for hk in range(num_kv_heads) for t in range(layout[r].q_len)}
    assert set(count) == want and all(v == 1 for v in count.values())
