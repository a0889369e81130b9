"""C ABI on the CPU: the library loads, exports what include/pkv.h declares,
and its host planner agrees bit for bit with the oracle's write slots,
permutation and restated tiling policy.  Error paths are forced from the host;
no call here touches a GPU."""
import os
import re

import numpy as np
import pytest

import oracle
import synth

pkv = pytest.importorskip("paged_kv_attention_plan_amd.pkv",
                          reason="libpkv.so not built (python -m paged_kv_attention_plan_amd.build)")

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pkv.h")


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text))
    assert declared, "no declarations found"
    import ctypes
    lib = ctypes.CDLL(pkv.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} is declared in pkv.h but not exported"
    assert declared <= set(pkv.EXPORTED)


def _params(w, kind, num_cus=4, **kw):
    return pkv.plan_params(kind, num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                           head_dim=w.head_dim, page_size=w.page_size, max_pages=w.max_pages,
                           causal=w.causal, window_left=w.window_left,
                           max_prefill_rows=w.max_prefill_rows, num_cus=num_cus, **kw)


def _layout(w):
    return oracle.decode_csr(w.page_size, w.kv_indptr, w.kv_indices, w.last_page_len,
                             max_pages=w.max_pages, qo_indptr=w.qo_indptr)


DECODE_CASES = [
    dict(seed=40, page_size=16, head_dim=64, window_left=-1, num_cus=1, wpc=4, mcp=1),
    dict(seed=41, page_size=1, head_dim=128, window_left=-1, num_cus=2, wpc=8, mcp=2),
    dict(seed=42, page_size=4, head_dim=64, window_left=17, num_cus=1, wpc=2, mcp=1),
    dict(seed=43, page_size=32, head_dim=128, window_left=0, num_cus=256, wpc=0, mcp=0),
    dict(seed=44, page_size=16, head_dim=128, window_left=-1, num_cus=3, wpc=0, mcp=1),
]


@pytest.mark.parametrize("c", DECODE_CASES, ids=lambda c: f"s{c['seed']}")
def test_decode_plan_matches_policy(c):
    w = synth.random_case(c["seed"], kind="decode", batch=7, head_dim=c["head_dim"],
                          page_size=c["page_size"], max_kv=300, window_left=c["window_left"])
    plan = pkv.plan_create(_params(w, "decode", num_cus=c["num_cus"], decode_waves_per_cu=c["wpc"],
                                   decode_min_chunk_pages=c["mcp"]),
                           None, w.kv_indptr, w.kv_indices, w.last_page_len)
    lay = _layout(w)
    rows = list(range(w.batch))
    tiles, merges, cap, n_slots, work = oracle.decode_policy(
        lay, rows, page_size=w.page_size, num_kv_heads=w.num_kv_heads, window_left=w.window_left,
        num_cus=c["num_cus"], qo_indptr=w.qo_indptr, kv_indptr=w.kv_indptr,
        group=w.num_qo_heads // w.num_kv_heads, waves_per_cu=c["wpc"],
        min_chunk_pages=c["mcp"] or 8)
    got = [tuple(int(x) for x in t) for t in plan.decode_tiles()]
    assert got == tiles
    assert [tuple(int(x) for x in m) for m in plan.merges()] == merges
    info = plan.info()
    assert info["worker_pages"] == cap and info["partial_slots"] == n_slots
    assert info["decode_workers"] == len(work) - 1
    img = plan.metadata()
    off = info["off_decode_work"]
    assert list(img[off:off + 4 * len(work)].view(np.int32)) == work
    oracle.check_decode_cover(got, merges, lay, rows, num_kv_heads=w.num_kv_heads,
                              window_left=w.window_left, n_slots=n_slots)
    slots = oracle.write_slots(w.page_size, w.kv_indptr, w.kv_indices, w.last_page_len)
    assert np.array_equal(plan.write_slots(), slots)
    # workspace covers metadata plus fp32 partials of every slot
    g = w.num_qo_heads // w.num_kv_heads
    assert info["workspace_bytes"] >= info["meta_bytes"] + n_slots * g * (w.head_dim + 1) * 4


@pytest.mark.parametrize("seed,hq,hk,num_cus,wpc", [(50, 32, 8, 256, 0), (51, 64, 8, 256, 0),
                                                   (52, 12, 3, 17, 4), (53, 8, 8, 64, 16)])
def test_decode_workers_are_balanced(seed, hq, hk, num_cus, wpc):
    """Every decode worker's share (its pages plus 2 per piece) lies within one
    piece cost and one page of the capacity, except the last worker's; no more
    workers than num_cus * waves_per_cu / Hk; each worker holds at most one
    piece of a row."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(1, 5000, size=int(rng.integers(20, 200)))
    w = synth.from_lengths(f"bal{seed}", "decode", kv, np.ones_like(kv), num_qo_heads=hq,
                           num_kv_heads=hk, head_dim=128, page_size=16, seed=seed,
                           layout_only=True)
    plan = pkv.plan_create(_params(w, "decode", num_cus=num_cus, decode_waves_per_cu=wpc),
                           None, w.kv_indptr, w.kv_indices, w.last_page_len)
    info = plan.info()
    g = hq // hk
    W = max(1, num_cus * (wpc or (16 if g == 8 else 4)) // hk)
    n_w, cap = info["decode_workers"], info["worker_pages"]
    assert 1 <= n_w <= W
    img = plan.metadata()
    work = img[info["off_decode_work"]:info["off_decode_work"] + 4 * (n_w + 1)].view(np.int32)
    tiles = plan.decode_tiles()
    pages = [-(-(int(t["kv_end"]) - int(t["kv_start"] // 16 * 16)) // 16) for t in tiles[::hk]]
    rows = [int(t["row"]) for t in tiles[::hk]]
    loads = []
    for k in range(n_w):
        ps = range(work[k], work[k + 1])
        assert len({rows[p] for p in ps}) == len(ps)
        loads.append(sum(pages[p] + 2 for p in ps))
    assert max(loads) <= cap
    assert min(loads[:-1], default=cap) >= cap - 2 - 1
    assert sum(pages) == sum(-(-int(n) // 16) for n in kv)


@pytest.mark.parametrize("causal,window_left,hq,hk,ps", [
    (True, -1, 8, 2, 4), (True, 6, 4, 4, 16), (False, -1, 8, 1, 1), (False, 9, 2, 1, 8),
    (True, -1, 16, 2, 64), (True, -1, 6, 2, 16), (True, 7, 24, 2, 8)])
def test_prefill_plan_matches_policy(causal, window_left, hq, hk, ps):
    w = synth.random_case(50, kind="prefill", batch=6, num_qo_heads=hq, num_kv_heads=hk,
                          head_dim=64, page_size=ps, max_kv=200, causal=causal,
                          window_left=window_left)
    plan = pkv.plan_create(_params(w, "prefill"), w.qo_indptr, w.kv_indptr, w.kv_indices,
                           w.last_page_len)
    lay = _layout(w)
    rows = [r for r in range(w.batch) if lay[r].q_len >= 1]
    want = oracle.prefill_policy(lay, rows, num_qo_heads=hq, num_kv_heads=hk, causal=causal,
                                 window_left=window_left, qo_indptr=w.qo_indptr,
                                 kv_indptr=w.kv_indptr)
    got = [tuple(int(x) for x in t)[:10] for t in plan.prefill_tiles()]
    assert got == want
    oracle.check_prefill_cover(got, lay, rows, num_kv_heads=hk, causal=causal,
                               window_left=window_left)
    slots = oracle.write_slots(ps, w.kv_indptr, w.kv_indices, w.last_page_len, qo_indptr=w.qo_indptr)
    assert np.array_equal(plan.write_slots(), slots)
    assert len(plan.decode_tiles()) == 0 and len(plan.permutation()) == 0


def test_mixed_plan_rows_and_permutation():
    w = synth.make_workload("mixed_window", scale_rows=12)
    plan = pkv.plan_create(_params(w, "mixed"), w.qo_indptr, w.kv_indptr, w.kv_indices,
                           w.last_page_len)
    dec, pre, perm = oracle.mixed_permutation(w.qo_indptr, max_prefill_rows=w.max_prefill_rows)
    assert np.array_equal(plan.permutation(), perm)
    info = plan.info()
    assert info["decode_rows"] == len(dec) and info["prompt_rows"] == len(pre)
    assert sorted({int(t["row"]) for t in plan.decode_tiles()}) == list(dec)
    assert sorted({int(t["row"]) for t in plan.prefill_tiles()}) == list(pre)
    lay = _layout(w)
    tiles, merges, cap, n_slots, work = oracle.decode_policy(
        lay, list(dec), page_size=w.page_size, num_kv_heads=w.num_kv_heads,
        window_left=w.window_left, num_cus=4, qo_indptr=w.qo_indptr, kv_indptr=w.kv_indptr,
        group=w.num_qo_heads // w.num_kv_heads)
    assert [tuple(int(x) for x in t) for t in plan.decode_tiles()] == tiles
    want = oracle.prefill_policy(lay, list(pre), num_qo_heads=w.num_qo_heads,
                                 num_kv_heads=w.num_kv_heads, causal=True,
                                 window_left=w.window_left, qo_indptr=w.qo_indptr,
                                 kv_indptr=w.kv_indptr)
    assert [tuple(int(x) for x in t)[:10] for t in plan.prefill_tiles()] == want


@pytest.mark.parametrize("name", ["tiny_decode", "gqa_decode"])
def test_full_size_decode_plans_cover(name):
    w = synth.make_workload(name) if name == "tiny_decode" else _lengths_only(name)
    plan = pkv.plan_create(_params(w, "decode", num_cus=256), None, w.kv_indptr, w.kv_indices,
                           w.last_page_len)
    lay = _layout(w)
    rows = list(range(w.batch))
    info = plan.info()
    got = [tuple(int(x) for x in t) for t in plan.decode_tiles()]
    oracle.check_decode_cover(got, [tuple(int(x) for x in m) for m in plan.merges()], lay, rows,
                              num_kv_heads=w.num_kv_heads, window_left=w.window_left,
                              n_slots=info["partial_slots"])


def _lengths_only(name):
    """The page table of a full-size workload without filling the pool."""
    k = synth.CONFIG_NAMES.index(name) + 1
    rng = np.random.default_rng(1000 + k)
    kv = rng.integers(512, 4097, size=128)
    npages = (kv + 15) // 16
    ids = rng.permutation(40000)[:npages.sum()].astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int32)
    class W: pass
    w = W()
    w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size = 32, 8, 128, 16
    w.max_pages, w.causal, w.window_left, w.max_prefill_rows = 40000, True, -1, 0
    w.kv_indptr, w.kv_indices = indptr, ids
    w.last_page_len = (((kv - 1) % 16) + 1).astype(np.int32)
    w.qo_indptr = np.arange(129)
    w.batch = 128
    return w


# ---- error paths ----

def _tiny():
    return synth.random_case(60, kind="decode", batch=3, page_size=4, head_dim=64, max_kv=20)


def _err(fn):
    with pytest.raises(pkv.PkvError) as ei:
        fn()
    return ei.value.status


def test_error_prefill_group_must_divide_tile_pairs():
    """Prefill tiles hold 192 (query head, token) pairs, so the GQA group
    num_qo_heads / num_kv_heads must divide 192: 3 and 64 do, 128 does not."""
    for hq, hk, ok in ((6, 2, True), (64, 1, True), (128, 1, False), (5, 1, False)):
        w = synth.random_case(51, kind="prefill", batch=2, num_qo_heads=hq, num_kv_heads=hk,
                              head_dim=64, page_size=16, max_kv=40)
        mk = lambda: pkv.plan_create(_params(w, "prefill"), w.qo_indptr, w.kv_indptr,
                                     w.kv_indices, w.last_page_len)
        if ok:
            mk()
        else:
            assert _err(mk) == pkv.E_UNSUPPORTED


def test_errors_unsupported_head_dim_and_page_size():
    w = _tiny()
    p = _params(w, "decode")
    p.head_dim = 96
    assert _err(lambda: pkv.plan_create(p, None, w.kv_indptr, w.kv_indices, w.last_page_len)) == pkv.E_UNSUPPORTED
    p = _params(w, "decode")
    p.page_size = 12
    assert _err(lambda: pkv.plan_create(p, None, w.kv_indptr, w.kv_indices, w.last_page_len)) == pkv.E_UNSUPPORTED


def test_error_page_over_2gib():
    """Pages are addressed with 32-bit offsets: 2 * page_size * Hk * D * 2 bytes
    must stay under 2 GiB (page 256, D 128: Hk below 16384)."""
    w = _tiny()
    p = _params(w, "decode")
    p.page_size, p.head_dim = 256, 128
    p.num_kv_heads, p.num_qo_heads = 16384, 16384
    assert _err(lambda: pkv.plan_create(p, None, w.kv_indptr, w.kv_indices, w.last_page_len)) == pkv.E_UNSUPPORTED
    assert "2 GiB" in pkv._lib.pkv_last_error().decode()
    p.num_kv_heads, p.num_qo_heads = 16383, 16383
    pkv.plan_create(p, None, w.kv_indptr, w.kv_indices, w.last_page_len)


@pytest.mark.parametrize("bad", ["lpl0", "lpl_big", "no_pages", "page_oob", "kv_lens", "heads"])
def test_errors_invalid_page_table(bad):
    w = _tiny()
    ind, idx, lpl = w.kv_indptr.copy(), w.kv_indices.copy(), w.last_page_len.copy()
    kv_lens = None
    p = _params(w, "decode")
    if bad == "lpl0":
        lpl[0] = 0
    if bad == "lpl_big":
        lpl[1] = 5
    if bad == "no_pages":
        ind[1] = ind[0]
    if bad == "page_oob":
        idx[0] = w.max_pages
    if bad == "kv_lens":
        kv_lens = w.kv_len.copy()
        kv_lens[2] += 1
    if bad == "heads":
        p.num_qo_heads = 3
    st = _err(lambda: pkv.plan_create(p, None, ind, idx, lpl, kv_lens))
    assert st == pkv.E_INVALID


def test_error_query_longer_than_kv():
    w = synth.random_case(61, kind="prefill", batch=2, page_size=4, head_dim=64, max_kv=20)
    qo = w.qo_indptr.copy()
    qo[1:] += 100
    assert _err(lambda: pkv.plan_create(_params(w, "prefill"), qo, w.kv_indptr, w.kv_indices,
                                        w.last_page_len)) == pkv.E_INVALID


def test_error_capacity_too_many_prompt_rows():
    w = synth.make_workload("mixed_window", scale_rows=6)
    p = _params(w, "mixed")
    p.max_prefill_rows = 3
    assert _err(lambda: pkv.plan_create(p, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                        w.last_page_len)) == pkv.E_CAPACITY


def test_error_conflicting_write_slots():
    # two rows sharing their last page: both new tokens land on one slot
    ind = np.array([0, 2, 4], dtype=np.int32)
    idx = np.array([0, 2, 1, 2], dtype=np.int32)
    lpl = np.array([3, 3], dtype=np.int32)
    p = pkv.plan_params("decode", num_qo_heads=2, num_kv_heads=1, head_dim=64, page_size=4,
                        max_pages=4, num_cus=1)
    assert _err(lambda: pkv.plan_create(p, None, ind, idx, lpl)) == pkv.E_CONFLICT


@pytest.mark.parametrize("seed", range(16))
def test_write_slot_conflicts_match_brute_force(seed):
    """The planner rejects a step with PKV_E_CONFLICT exactly when two of its
    query tokens' write slots (page * ps + offset, kv.plan) coincide, checked
    here with a set of all slots.  Rows draw pages from a small pool, with
    repeats inside a row and across rows, so both outcomes occur."""
    rng = np.random.default_rng(300 + seed)
    ps = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(2, 7))
    kv = rng.integers(1, 6 * ps + 1, size=B)
    ql = np.array([rng.integers(1, k + 1) for k in kv])
    npg = (kv + ps - 1) // ps
    pool = int(rng.integers(max(2, int(npg.max())), 8 * int(npg.sum()) + 3))
    idx = rng.integers(0, pool, size=int(npg.sum())).astype(np.int32)
    ind = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    lpl = ((kv - 1) % ps + 1).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    slots = []
    for r in range(B):
        for p_ in range(int(kv[r] - ql[r]), int(kv[r])):
            slots.append(int(idx[ind[r] + p_ // ps]) * ps + p_ % ps)
    dup = len(set(slots)) < len(slots)
    p = pkv.plan_params("prefill", num_qo_heads=2, num_kv_heads=1, head_dim=64, page_size=ps,
                        max_pages=pool, num_cus=1)
    if dup:
        assert _err(lambda: pkv.plan_create(p, qo, ind, idx, lpl)) == pkv.E_CONFLICT
    else:
        plan = pkv.plan_create(p, qo, ind, idx, lpl)
        assert list(plan.write_slots()) == slots


def test_shared_pages_for_reading_are_allowed():
    ind = np.array([0, 2, 4], dtype=np.int32)
    idx = np.array([0, 2, 1, 3], dtype=np.int32)  # page 0..: rows share nothing but may
    idx[2] = 0                                      # row 1 reads row 0's first page
    lpl = np.array([3, 2], dtype=np.int32)
    p = pkv.plan_params("decode", num_qo_heads=2, num_kv_heads=1, head_dim=64, page_size=4,
                        max_pages=4, num_cus=1)
    pkv.plan_create(p, None, ind, idx, lpl)


def test_error_qo_indptr_presence():
    w = _tiny()
    assert _err(lambda: pkv.plan_create(_params(w, "decode"), w.qo_indptr, w.kv_indptr,
                                        w.kv_indices, w.last_page_len)) == pkv.E_INVALID
    assert _err(lambda: pkv.plan_create(_params(w, "prefill"), None, w.kv_indptr, w.kv_indices,
                                        w.last_page_len)) == pkv.E_INVALID


class _FakeTensor:
    """Stands in for a device tensor: the ABI rejects these calls before any
    device access, so the pointer is never dereferenced."""
    is_cuda = True

    def __init__(self, nbytes):
        self._n = nbytes

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 4096

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def test_error_workspace_too_small_reports_bytes():
    w = _tiny()
    plan = pkv.plan_create(_params(w, "decode"), None, w.kv_indptr, w.kv_indices, w.last_page_len)
    with pytest.raises(pkv.PkvError) as ei:
        pkv.plan_upload(plan, _FakeTensor(plan.ws_bytes - 1), stream=0)
    assert ei.value.status == pkv.E_WORKSPACE
    assert str(plan.ws_bytes) in ei.value.message


def test_error_run_before_upload():
    w = _tiny()
    plan = pkv.plan_create(_params(w, "decode"), None, w.kv_indptr, w.kv_indices, w.last_page_len)
    import ctypes
    st = pkv._lib.pkv_run(plan.handle, ctypes.c_void_p(4096), ctypes.c_void_p(4096),
                          ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), plan.ws_bytes,
                          ctypes.c_void_p(0))
    assert st == pkv.E_STATE


def test_error_run_append_before_upload():
    w = _tiny()
    plan = pkv.plan_create(_params(w, "decode"), None, w.kv_indptr, w.kv_indices, w.last_page_len)
    import ctypes
    v = ctypes.c_void_p(4096)
    st = pkv._lib.pkv_run_append(plan.handle, v, v, v, v, v, None, v, plan.ws_bytes,
                                 ctypes.c_void_p(0))
    assert st == pkv.E_STATE
    st = pkv._lib.pkv_run_append(None, v, v, v, v, v, None, v, plan.ws_bytes, ctypes.c_void_p(0))
    assert st == pkv.E_INVALID


def test_plan_update_reuses_handle_and_keeps_old_plan_on_error():
    w = _tiny()
    p = _params(w, "decode")
    p.max_pages = 1000
    plan = pkv.plan_create(p, None, w.kv_indptr, w.kv_indices, w.last_page_len)
    before = plan.decode_tiles()
    w2 = synth.random_case(62, kind="decode", batch=5, page_size=4, head_dim=64, max_kv=40)
    bad = w2.last_page_len.copy()
    bad[0] = 0
    with pytest.raises(pkv.PkvError):
        pkv.plan_update(plan, None, w2.kv_indptr, w2.kv_indices, bad)
    assert np.array_equal(plan.decode_tiles(), before)
    pkv.plan_update(plan, None, w2.kv_indptr, w2.kv_indices, w2.last_page_len)
    assert plan.info()["batch"] == 5


def test_empty_batch():
    p = pkv.plan_params("prefill", num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                        max_pages=8, num_cus=4)
    plan = pkv.plan_create(p, np.zeros(1), np.zeros(1), np.zeros(0), np.zeros(0))
    assert plan.info()["total_q"] == 0 and len(plan.prefill_tiles()) == 0
    assert plan.ws_bytes > 0


# ---- graph-static plans ----

def _static_params(w, kind, B=16, T=1024, E=4096, max_pages=1000, **kw):
    p = _params(w, kind, static_max_batch=B, static_max_tokens=T, static_max_page_entries=E, **kw)
    p.max_pages = max_pages
    return p


@pytest.mark.parametrize("kind", ["decode", "prefill", "mixed"])
def test_static_plan_layout_is_fixed_across_replans(kind):
    """The workspace layout of a graph-static plan depends on its capacities
    only, and its tiles are those of the ordinary plan of the same step."""
    seeds = [81, 82, 83]
    plan = sizes = None
    for sd in seeds:
        w = synth.random_case(sd, kind="decode" if kind == "decode" else "prefill", batch=6,
                              page_size=4, head_dim=64, max_kv=120)
        w.max_prefill_rows = 6
        qo = None if kind == "decode" else w.qo_indptr
        p = _static_params(w, kind)
        if plan is None:
            plan = pkv.plan_create(p, qo, w.kv_indptr, w.kv_indices, w.last_page_len)
        else:
            pkv.plan_update(plan, qo, w.kv_indptr, w.kv_indices, w.last_page_len)
        info = plan.info()
        now = (info["meta_bytes"], info["workspace_bytes"], plan.ws_bytes)
        assert sizes is None or now == sizes
        sizes = now
        p0 = _params(w, kind)
        p0.max_pages = 1000
        ref = pkv.plan_create(p0, qo, w.kv_indptr, w.kv_indices, w.last_page_len)
        assert np.array_equal(plan.decode_tiles(), ref.decode_tiles())
        assert np.array_equal(plan.prefill_tiles(), ref.prefill_tiles())
        assert np.array_equal(plan.merges(), ref.merges())
        assert np.array_equal(plan.write_slots(), ref.write_slots())


def test_static_plan_capacity_errors():
    w = synth.random_case(84, kind="decode", batch=6, page_size=4, head_dim=64, max_kv=120)
    with pytest.raises(pkv.PkvError, match="graph-static capacities"):
        pkv.plan_create(_static_params(w, "decode", B=5), None, w.kv_indptr,
                        w.kv_indices, w.last_page_len)
    with pytest.raises(pkv.PkvError, match="graph-static capacities"):
        pkv.plan_create(_static_params(w, "decode", E=3), None, w.kv_indptr,
                        w.kv_indices, w.last_page_len)
    plan = pkv.plan_create(_static_params(w, "decode"), None, w.kv_indptr,
                           w.kv_indices, w.last_page_len)
    w2 = synth.random_case(85, kind="decode", batch=20, page_size=4, head_dim=64, max_kv=120)
    try:
        pkv.plan_update(plan, None, w2.kv_indptr, w2.kv_indices, w2.last_page_len)
        raise AssertionError("expected a capacity error")
    except pkv.PkvError as e:
        assert e.status == pkv.E_CAPACITY
    # partial capacities and dense static plans are rejected
    p = _params(w, "decode", static_max_batch=4)
    with pytest.raises(pkv.PkvError, match="all be >= 1"):
        pkv.plan_create(p, None, w.kv_indptr, w.kv_indices, w.last_page_len)
    pd = pkv.plan_params("dense", num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=4,
                         max_pages=10, num_cus=4, static_max_batch=1, static_max_tokens=1,
                         static_max_page_entries=1)
    with pytest.raises(pkv.PkvError, match="graph-static"):
        pkv.dense_plan_create(pd, [0, 1], [0, 2])
