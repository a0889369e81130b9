"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every output element is compared with the oracle.  The five full-size
workloads run in the launch configuration the benchmark times and are held to
max |out - ref| <= 1e-2 and max |lse - ref| <= 1e-3 on every element.  The
small edge cases add half a bf16 ulp of ref where |ref| >= 2 (the bf16
output's own rounding; see gpu_common).  Write slots and appended bytes are
bit-exact.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, gpu_run, oracle_all, oracle_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def _full_oracle(w):
    wc = w.to("cpu")
    return oracle.attention(wc.q, wc.cache, w.page_size, w.kv_indptr, w.kv_indices,
                            w.last_page_len, num_qo_heads=w.num_qo_heads,
                            num_kv_heads=w.num_kv_heads,
                            qo_indptr=None if w.kind == "decode" else w.qo_indptr,
                            causal=w.causal, window_left=w.window_left)


def test_tiny_decode_matches_golden_and_oracle(pkv, gpu):
    say("case tiny_decode (4 rows, Hq 4 / Hk 2, D 64, ps 16)")
    w = synth.make_workload("tiny_decode").to(gpu)
    out, lse, plan, _ = gpu_run(pkv, w)
    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_decode.json")))
    compare(out, lse, np.array(doc["out"]), np.array(doc["lse"]), "tiny_decode vs golden")
    ref_o, ref_l = _full_oracle(w)
    compare(out, lse, ref_o, ref_l, "tiny_decode vs oracle")
    assert list(plan.write_slots()) == doc["write_slots"]


DECODE = [
    # (seed, head_dim, Hq, Hk, page_size, window, stale, force_split)
    (100, 64, 4, 2, 16, -1, "nan", False),
    (101, 128, 32, 8, 16, -1, "nan", True),
    (102, 128, 8, 8, 1, -1, "nan", True),
    (103, 64, 16, 2, 64, 37, "nan", True),
    (104, 128, 16, 16, 32, 0, "nan", False),
    (105, 64, 8, 4, 4, 100, "zero", True),
    (106, 128, 16, 2, 256, -1, "nan", True),
    (107, 64, 2, 1, 8, -1, "nan", True),
    # KV head counts that are not a multiple of the 4 waves of a workgroup, so a
    # worker's waves straddle workgroups; group 8 without splits
    (108, 128, 12, 3, 16, -1, "nan", True),
    (109, 128, 40, 5, 8, 50, "nan", False),
    (110, 64, 6, 3, 16, -1, "nan", True),
    (111, 128, 64, 8, 16, -1, "nan", False),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"s{c[0]}-D{c[1]}-g{c[2]//c[3]}-ps{c[4]}-w{c[5]}")
def test_decode_small(pkv, gpu, case):
    seed, D, hq, hk, ps, wl, stale, split = case
    say(f"case decode seed={seed} D={D} Hq={hq} Hk={hk} ps={ps} window={wl} split={split}")
    w = synth.random_case(seed, kind="decode", batch=9, num_qo_heads=hq, num_kv_heads=hk,
                          head_dim=D, page_size=ps, max_kv=700, window_left=wl, stale=stale,
                          device=gpu)
    # a large tile budget with 1-page chunks makes the planner cut rows into chunks
    kw = dict(num_cus=64, decode_waves_per_cu=16, decode_min_chunk_pages=1) if split else {}
    out, lse, plan, _ = gpu_run(pkv, w, **kw)
    if split:
        assert len(plan.merges()) > 0
    ref_o, ref_l = _full_oracle(w)
    compare(out, lse, ref_o, ref_l, f"decode s{seed}")


def _random_decode_shapes(n=16, seed=4141):
    """Seeded decode shapes across head dims, GQA groups, KV head counts that do
    and do not fill a 4-wave workgroup, page sizes 1..256, windows, stale data
    and forced splits."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        hk = int(rng.choice([1, 2, 3, 4, 5, 8]))
        ps = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256]))
        wl = int(rng.choice([-1, -1, 0, 9, 200]))
        out.append((150 + k, D, g * hk, hk, ps, wl, "nan" if k % 2 else "zero", bool(k % 3)))
    return out


@pytest.mark.parametrize("case", _random_decode_shapes(),
                         ids=lambda c: f"s{c[0]}-D{c[1]}-g{c[2]//c[3]}-ps{c[4]}-w{c[5]}-split{int(c[7])}")
def test_decode_random_shapes(pkv, gpu, case):
    seed, D, hq, hk, ps, wl, stale, split = case
    say(f"case decode sweep seed={seed} D={D} Hq={hq} Hk={hk} ps={ps} window={wl} split={split}")
    w = synth.random_case(seed, kind="decode", batch=7, num_qo_heads=hq, num_kv_heads=hk,
                          head_dim=D, page_size=ps, max_kv=900, window_left=wl, stale=stale,
                          device=gpu)
    kw = dict(num_cus=32, decode_waves_per_cu=16, decode_min_chunk_pages=1) if split else {}
    out, lse, plan, _ = gpu_run(pkv, w, **kw)
    ref_o, ref_l = _full_oracle(w)
    compare(out, lse, ref_o, ref_l, f"decode sweep s{seed}")


PREFILL = [
    # (seed, head_dim, Hq, Hk, page_size, causal, window, stale)
    (200, 128, 32, 8, 16, True, -1, "nan"),
    (201, 64, 4, 4, 16, True, -1, "nan"),
    (202, 128, 8, 1, 1, True, 5, "nan"),
    (203, 64, 16, 2, 32, False, -1, "nan"),
    (204, 128, 4, 2, 64, False, 40, "nan"),
    (205, 64, 8, 8, 4, True, 0, "zero"),
    (206, 128, 16, 16, 16, True, 300, "nan"),
    # group sizes whose query blocks straddle heads inside a 16-lane block
    (207, 128, 6, 2, 16, True, -1, "nan"),     # g 3: 64 tokens per tile
    (208, 128, 32, 2, 16, True, 100, "nan"),   # g 16: 12 tokens per tile
    (209, 64, 24, 2, 8, True, -1, "nan"),      # g 12, pages of 8 (per-lane page ids)
    (210, 128, 64, 1, 32, False, -1, "nan"),   # g 64: 3 tokens per tile
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: f"s{c[0]}-D{c[1]}-g{c[2]//c[3]}-ps{c[4]}-c{int(c[5])}-w{c[6]}")
def test_prefill_small(pkv, gpu, case):
    seed, D, hq, hk, ps, causal, wl, stale = case
    say(f"case prefill seed={seed} D={D} Hq={hq} Hk={hk} ps={ps} causal={causal} window={wl}")
    w = synth.random_case(seed, kind="prefill", batch=6, num_qo_heads=hq, num_kv_heads=hk,
                          head_dim=D, page_size=ps, max_kv=600, causal=causal, window_left=wl,
                          stale=stale, device=gpu)
    out, lse, plan, _ = gpu_run(pkv, w)
    ref_o, ref_l = _full_oracle(w)
    compare(out, lse, ref_o, ref_l, f"prefill s{seed}")


def _random_prefill_shapes(n=16, seed=4242):
    """Seeded prefill shapes across head dims, GQA groups (including ones that
    straddle heads inside a 16-lane query block), page sizes, masks and stale data."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        hk = int(rng.choice([1, 2, 4])) if g <= 8 else 1
        ps = int(rng.choice([1, 2, 8, 16, 32, 64, 128]))
        causal = bool(rng.integers(0, 2))
        wl = int(rng.choice([-1, -1, 0, 17, 130]))
        out.append((300 + k, D, g * hk, hk, ps, causal, wl, "nan" if k % 2 else "zero"))
    return out


@pytest.mark.parametrize("case", _random_prefill_shapes(),
                         ids=lambda c: f"s{c[0]}-D{c[1]}-g{c[2]//c[3]}-ps{c[4]}-c{int(c[5])}-w{c[6]}")
def test_prefill_random_shapes(pkv, gpu, case):
    seed, D, hq, hk, ps, causal, wl, stale = case
    say(f"case prefill sweep seed={seed} D={D} Hq={hq} Hk={hk} ps={ps} causal={causal} window={wl}")
    w = synth.random_case(seed, kind="prefill", batch=5, num_qo_heads=hq, num_kv_heads=hk,
                          head_dim=D, page_size=ps, max_kv=400, causal=causal, window_left=wl,
                          stale=stale, device=gpu)
    out, lse, plan, _ = gpu_run(pkv, w)
    ref_o, ref_l = _full_oracle(w)
    compare(out, lse, ref_o, ref_l, f"prefill sweep s{seed}")


def test_mixed_small(pkv, gpu):
    say("case mixed_window cut to 12 decode rows + 4 prompt rows")
    w = synth.make_workload("mixed_window", scale_rows=12, device=gpu, stale="nan")
    out, lse, plan, _ = gpu_run(pkv, w)
    ref_o, ref_l = _full_oracle(w)
    compare(out, lse, ref_o, ref_l, "mixed small")


def test_decode_equals_prefill_one_token(pkv, gpu):
    say("case decode vs prefill with one query per row")
    w = synth.random_case(300, kind="decode", batch=7, num_qo_heads=8, num_kv_heads=2,
                          head_dim=128, page_size=16, max_kv=400, device=gpu)
    o1, l1, _, _ = gpu_run(pkv, w)
    o2, l2, _, _ = gpu_run(pkv, w, kind="prefill")
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_append_kv_bit_exact(pkv, gpu):
    say("case append_kv: decode rows, slots at last_page_len - 1")
    w = synth.random_case(310, kind="decode", batch=11, num_qo_heads=8, num_kv_heads=4,
                          head_dim=128, page_size=16, max_kv=300, new_tokens=True, device=gpu)
    before = w.cache.clone()
    p = pkv.plan_create(pkv.plan_params("decode", num_qo_heads=8, num_kv_heads=4, head_dim=128,
                                        page_size=16, max_pages=w.max_pages),
                        None, w.kv_indptr, w.kv_indices, w.last_page_len)
    ws = torch.empty(p.ws_bytes, dtype=torch.uint8, device=gpu)
    pkv.plan_upload(p, ws)
    pkv.append_kv(p, w.k_new, w.v_new, w.cache, ws)
    torch.cuda.synchronize()
    slots = oracle.write_slots(16, w.kv_indptr, w.kv_indices, w.last_page_len)
    assert np.array_equal(p.write_slots(), slots)
    bits = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    want = oracle.apply_append(bits(before), slots, bits(w.k_new), bits(w.v_new), 16)
    assert np.array_equal(bits(w.cache), want)


def test_append_prefill_tokens_bit_exact(pkv, gpu):
    say("case append_kv: ragged prefill tokens")
    w = synth.random_case(311, kind="prefill", batch=5, num_qo_heads=4, num_kv_heads=2,
                          head_dim=64, page_size=8, max_kv=200, new_tokens=True, device=gpu)
    before = w.cache.clone()
    _, _, p, ws = gpu_run(pkv, w, append=True)
    slots = oracle.write_slots(8, w.kv_indptr, w.kv_indices, w.last_page_len, qo_indptr=w.qo_indptr)
    bits = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    want = oracle.apply_append(bits(before), slots, bits(w.k_new), bits(w.v_new), 8)
    assert np.array_equal(bits(w.cache), want)


def test_page_relabelling_is_bit_identical(pkv, gpu):
    say("case page relabelling")
    w = synth.random_case(320, kind="prefill", batch=5, num_qo_heads=8, num_kv_heads=2,
                          head_dim=128, page_size=16, max_kv=500, device=gpu, extra_pages=9)
    o1, l1, _, _ = gpu_run(pkv, w)
    perm = np.random.default_rng(5).permutation(w.max_pages)
    cache2 = torch.empty_like(w.cache)
    cache2[torch.from_numpy(perm).to(gpu)] = w.cache
    w2 = synth.Workload(**{**w.__dict__, "cache": cache2,
                           "kv_indices": perm[w.kv_indices].astype(np.int32)})
    o2, l2, _, _ = gpu_run(pkv, w2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeat_runs_are_deterministic(pkv, gpu):
    say("case repeat determinism (split decode)")
    w = synth.random_case(330, kind="decode", batch=9, num_qo_heads=32, num_kv_heads=8,
                          head_dim=128, page_size=16, max_kv=900, device=gpu)
    kw = dict(num_cus=64, decode_waves_per_cu=16, decode_min_chunk_pages=1)
    o1, l1, p1, _ = gpu_run(pkv, w, **kw)
    o2, l2, _, _ = gpu_run(pkv, w, **kw)
    assert len(p1.merges()) > 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- full sizes, every element, flat bounds ----
# Each workload runs in the launch configuration the benchmark times (default
# plan parameters on the device's CU count), and every output element and LSE
# is compared with the oracle at max |out - ref| <= 1e-2, max |lse - ref| <= 1e-3.


def test_full_gqa_decode_with_append(pkv, gpu):
    say("case gqa_decode full size (128 rows, Hq 32 / Hk 8, D 128, ps 16, 40000-page pool) + append")
    w = synth.make_workload("gqa_decode", device=gpu)
    before = w.cache.clone()
    out, lse, plan, _ = gpu_run(pkv, w, append=True)
    # the appended tokens, bit for bit, and nothing else of the pool moved
    slots = oracle.write_slots(16, w.kv_indptr, w.kv_indices, w.last_page_len)
    assert np.array_equal(plan.write_slots(), slots)
    sl = torch.from_numpy(slots).to(gpu)
    page, off = sl // 16, sl % 16
    assert torch.equal(w.cache[page, 0, off], w.k_new) and torch.equal(w.cache[page, 1, off], w.v_new)
    before[page, 0, off] = w.k_new
    before[page, 1, off] = w.v_new
    assert torch.equal(before.view(torch.int16), w.cache.view(torch.int16))
    del before
    ref_o, ref_l = oracle_all(w)
    compare(out, lse, ref_o, ref_l, "gqa_decode full (all 128 rows)", flat=True)


def test_full_long_decode(pkv, gpu):
    say("case long_decode full size (8 rows, N in [32768, 131072], split-KV)")
    w = synth.make_workload("long_decode", device=gpu)
    out, lse, plan, _ = gpu_run(pkv, w)
    assert len(plan.merges()) > 0
    ref_o, ref_l = oracle_all(w)
    compare(out, lse, ref_o, ref_l, "long_decode full (all 8 rows)", flat=True)


def test_full_ragged_prefill(pkv, gpu):
    say("case ragged_prefill full size (16 rows, q 128..2048, prefix 0..4096)")
    w = synth.make_workload("ragged_prefill", device=gpu)
    out, lse, plan, _ = gpu_run(pkv, w)
    ref_o, ref_l = oracle_all(w)
    compare(out, lse, ref_o, ref_l, f"ragged_prefill full (all {w.total_q} tokens)", flat=True)


def test_full_mixed_window(pkv, gpu):
    say("case mixed_window full size (256 decode rows + 4 prompt rows, window 4096)")
    w = synth.make_workload("mixed_window", device=gpu)
    out, lse, plan, _ = gpu_run(pkv, w)
    dec, pre, perm = oracle.mixed_permutation(w.qo_indptr, max_prefill_rows=4)
    assert np.array_equal(plan.permutation(), perm)
    ref_o, ref_l = oracle_all(w)
    compare(out, lse, ref_o, ref_l, f"mixed_window full (all {w.total_q} tokens)", flat=True)
    dq = np.asarray(w.qo_indptr)[dec]
    compare(out[torch.from_numpy(dq.astype(np.int64)).to(gpu)], lse[torch.from_numpy(dq.astype(np.int64)).to(gpu)],
            ref_o[dq], ref_l[dq], "mixed_window decode rows", flat=True)
    compare(out[torch.from_numpy(perm.astype(np.int64)).to(gpu)], lse[torch.from_numpy(perm.astype(np.int64)).to(gpu)],
            ref_o[perm], ref_l[perm], "mixed_window prompt tokens", flat=True)
