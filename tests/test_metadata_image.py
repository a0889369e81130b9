"""The metadata image the kernels read (pkv_plan_metadata, the bytes the upload
copies into the workspace), decoded on the CPU the way the kernels decode it.

For every workload shape (full-size lengths, forced split-KV, graph-static and
dense plans) the image must agree with the public tile lists, and every index
a kernel derives from it must stay inside its buffer: the worker table gives
every decode wave a range of pieces inside the piece list; a piece's row
record gives its page base, query and partial slot for each KV head; its keys
lie in the row's pages; merges address existing partial slots; prefill tiles,
page indices and write slots are the planned ones; regions do not overlap and
fit the workspace.  No GPU is involved.
"""
import numpy as np
import pytest

import synth

pkv = pytest.importorskip("paged_kv_attention_plan_amd.pkv",
                          reason="libpkv.so not built (python -m paged_kv_attention_plan_amd.build)")

PIECE = np.dtype([("row", "<i4"), ("chunk", "<i4"), ("ks", "<i4"), ("ke", "<i4")])
DROW = np.dtype([("page_base", "<i4"), ("q_index", "<i4"), ("kv_len", "<i4"), ("slot0", "<i4"),
                 ("n_chunks", "<i4"), ("pad", "<i4", (3,))])
NROW = np.dtype([("cu_k", "<i4"), ("cu_q", "<i4"), ("prefix", "<i4"), ("fresh", "<i4"),
                 ("page_base", "<i4"), ("pad", "<i4", (3,))])


def _a256(x):
    return (x + 255) // 256 * 256


def _check(plan, kind, kv_indptr, kv_indices, last_page_len, qo_indptr, hk, g, d, ps,
           static_tokens=None):
    info = plan.info()
    img = plan.metadata()
    assert len(img) == info["meta_bytes"] and info["meta_bytes"] % 256 == 0
    hdr = img[:64].view(np.int64)
    n_dt, n_m, n_pt, n_idx, n_sl, n_slots, T, B = (int(x) for x in hdr)
    pub = plan.decode_tiles()
    assert n_m == len(plan.merges()) and n_pt == len(plan.prefill_tiles())
    assert n_idx == len(kv_indices) and T == info["total_q"] and B == info["batch"]
    assert n_slots == info["partial_slots"] and n_sl == len(plan.write_slots())
    # regions in order, each inside the metadata image
    offs = [info["off_dense_rows"], info["off_decode_rows"], info["off_decode_pieces"],
            info["off_decode_work"], info["off_merges"], info["off_prefill_tiles"],
            info["off_indices"]]
    assert offs[0] == 256 and offs == sorted(offs) and offs[-1] <= info["meta_bytes"]
    # the worker table, as the decode kernel's waves read it: worker w (Hk waves)
    # runs pieces [work[w], work[w + 1]); every piece belongs to one worker
    n_w = info["decode_workers"]
    assert (n_w + 1) * 4 <= offs[4] - offs[3]
    work = img[offs[3]:offs[3] + 4 * (n_w + 1)].view(np.int32)
    if n_dt:
        assert work[0] == 0 and work[-1] == n_dt and np.all(np.diff(work) >= 0)
    else:
        assert np.all(work == 0)
    # decode pieces through the row table, as the decode kernel reads them
    n_rows = (offs[2] - offs[1]) // DROW.itemsize
    rows = img[offs[1]:offs[1] + n_rows * DROW.itemsize].view(DROW)
    pieces = img[offs[2]:offs[2] + n_dt * PIECE.itemsize].view(PIECE)
    assert n_dt * PIECE.itemsize <= offs[3] - offs[2]
    assert len(pub) == n_dt * hk
    for t, pt in enumerate(pub):
        tm = pieces[t // hk]
        assert pt["kv_head"] == t % hk
        assert 0 <= tm["row"] < n_rows
        r = rows[tm["row"]]
        assert (r["page_base"], r["q_index"], r["kv_len"]) == (pt["page_base"], pt["q_index"], pt["kv_len"])
        assert (tm["ks"], tm["ke"]) == (pt["kv_start"], pt["kv_end"])
        assert 0 <= tm["chunk"] < r["n_chunks"]
        slot = r["slot0"] + pt["kv_head"] * r["n_chunks"] + tm["chunk"] if r["slot0"] >= 0 else -1
        assert slot == pt["out_slot"] and slot < n_slots
        assert 0 <= r["q_index"] < T
        assert 0 <= tm["ks"] < tm["ke"] <= r["kv_len"]
        row = int(pt["row"])
        first, last = r["page_base"] + tm["ks"] // ps, r["page_base"] + (tm["ke"] - 1) // ps
        assert kv_indptr[row] <= first and last < kv_indptr[row + 1]
    # merges, as the merge kernel reads them
    mer = img[offs[4]:offs[4] + n_m * 16].view(np.int32).reshape(-1, 4)
    assert n_m * 16 <= offs[5] - offs[4]
    assert np.array_equal(mer, plan.merges().view(np.int32).reshape(-1, 4))
    for q_index, head, base, n in mer:
        assert 0 <= q_index < T and 0 <= head < hk and 0 <= base and base + n <= n_slots and n >= 2
    # prefill tiles, page indices and write slots are the planned ones
    pre = img[offs[5]:offs[5] + n_pt * 48]
    assert n_pt * 48 <= offs[6] - offs[5]
    assert np.array_equal(pre, plan.prefill_tiles().view(np.uint8).reshape(-1))
    assert np.array_equal(img[offs[6]:offs[6] + 4 * n_idx].view(np.int32), kv_indices)
    slot_cap = static_tokens if static_tokens is not None else n_sl
    off_slots = info["meta_bytes"] - _a256(8 * slot_cap)
    assert off_slots >= offs[6] + 4 * n_idx
    assert np.array_equal(img[off_slots:off_slots + 8 * n_sl].view(np.int64), plan.write_slots())
    # partials fit the workspace
    need = _a256(n_slots * g * d * 4) + _a256(n_slots * g * 4)
    assert info["workspace_bytes"] >= info["meta_bytes"] + need


def _params(w, kind, **kw):
    return pkv.plan_params(kind, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                           head_dim=w.head_dim, page_size=w.page_size, max_pages=w.max_pages,
                           causal=w.causal, window_left=w.window_left,
                           max_prefill_rows=w.max_prefill_rows, num_cus=kw.pop("num_cus", 256), **kw)


def _run(w, kind, static=False, **kw):
    g = w.num_qo_heads // w.num_kv_heads
    if static:
        kw.update(static_max_batch=w.batch + 3, static_max_tokens=int(w.qo_indptr[-1]) + 17,
                  static_max_page_entries=len(w.kv_indices) + 100)
    qo = None if kind == "decode" else w.qo_indptr
    plan = pkv.plan_create(_params(w, kind, **kw), qo, w.kv_indptr, w.kv_indices, w.last_page_len)
    _check(plan, kind, w.kv_indptr, w.kv_indices, w.last_page_len, qo, w.num_kv_heads, g,
           w.head_dim, w.page_size,
           static_tokens=int(w.qo_indptr[-1]) + 17 if static else None)


def _layout(name):
    """A workload's page table and shapes without filling its cache."""
    return synth.make_workload(name, layout_only=True)


@pytest.mark.parametrize("name", ["gqa_decode", "long_decode", "ragged_prefill", "mixed_window"])
@pytest.mark.parametrize("static", [False, True])
def test_full_size_images(name, static):
    w = _layout(name)
    _run(w, w.kind, static=static)


@pytest.mark.parametrize("seed,kind,ps,wl", [(1201, "decode", 16, -1), (1202, "decode", 1, 9),
                                             (1203, "decode", 4, -1), (1204, "mixed", 32, 50),
                                             (1205, "prefill", 2, -1)])
@pytest.mark.parametrize("static", [False, True])
def test_forced_split_images(seed, kind, ps, wl, static):
    w = synth.random_case(seed, kind="decode" if kind == "decode" else "prefill", batch=11,
                          num_qo_heads=16, num_kv_heads=4, head_dim=64, page_size=ps, max_kv=700,
                          window_left=wl)
    if kind == "mixed":
        # three rows with several queries, the rest one query each
        ql = np.ones(w.batch, dtype=np.int64)
        ql[[1, 4, 7]] = np.minimum(w.kv_len[[1, 4, 7]], 40)
        w = synth.from_lengths("m", "mixed", w.kv_len, ql, num_qo_heads=16, num_kv_heads=4,
                               head_dim=64, page_size=ps, window_left=wl, seed=seed,
                               max_prefill_rows=3)
    _run(w, kind, static=static, num_cus=16, decode_waves_per_cu=8, decode_min_chunk_pages=1)


def test_dense_rows_image():
    rng = np.random.default_rng(7)
    B, ps = 9, 16
    L = rng.integers(0, 300, size=B)
    P = rng.integers(0, 500, size=B)
    cu_q = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(L + P)]).astype(np.int32)
    npages = (P + ps - 1) // ps + rng.integers(0, 3, size=B)
    ind = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    idx = rng.permutation(int(ind[-1]) + 50)[:int(ind[-1])].astype(np.int32)
    p = pkv.plan_params("dense", num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=ps,
                        max_pages=int(idx.max()) + 1, num_cus=8)
    plan = pkv.dense_plan_create(p, cu_q, cu_k, ind, idx)
    info = plan.info()
    img = plan.metadata()
    rows = img[info["off_dense_rows"]:info["off_dense_rows"] + B * NROW.itemsize].view(NROW)
    assert list(rows["cu_k"]) == list(cu_k[:-1]) and list(rows["cu_q"]) == list(cu_q[:-1])
    assert list(rows["prefix"]) == list(P) and list(rows["fresh"]) == list(L)
    assert list(rows["page_base"]) == list(ind[:-1])
    for r in range(B):  # the gather reads prefix pages inside the row's entries
        if P[r]:
            assert rows["page_base"][r] + (P[r] - 1) // ps < ind[r + 1]
    off = info["off_indices"]
    assert np.array_equal(img[off:off + 4 * len(idx)].view(np.int32), idx)
    pre = plan.prefill_tiles()
    assert np.array_equal(img[info["off_prefill_tiles"]:info["off_prefill_tiles"] + 48 * len(pre)],
                          pre.view(np.uint8).reshape(-1))
    for t in pre:  # a dense tile's keys are dense rows [cu_k, cu_k + kv_len) of its row
        r = int(t["row"])
        assert t["page_base"] == cu_k[r] and t["kv_len"] == cu_k[r + 1] - cu_k[r]
        assert 0 <= t["kv_lo"] <= t["kv_hi"] < t["kv_len"]
