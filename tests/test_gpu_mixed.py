"""The mixed step (attn.wrappers › FlashInferMixedWrapper: one-token rows on the
decode plan, prompt rows on the prefill plan, both in one step) on the GPU.

With page_size >= 16 a mixed plan runs its decode waves and its prefill tiles
in one launch; below that it launches them one after the other.  Either way
the output must be, bit for bit, what a decode plan over the one-token rows
and a prefill plan over the prompt rows give on the same bytes (the same
device code on the same pieces and tiles), and within tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import compare, gpu_run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv(gpu):
    from paged_kv_attention_plan_amd import pkv as mod
    return mod


def _sub(w, rows, kind):
    """The page table and packed q of a subset of w's rows, as a workload of
    the given kind over the same cache."""
    ind = [0]
    idx = []
    toks = []
    for r in rows:
        a, b = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        idx.extend(w.kv_indices[a:b])
        ind.append(ind[-1] + b - a)
        toks.extend(range(int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])))
    ql = np.array([int(w.q_len[r]) for r in rows])
    qo = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    t = torch.tensor(toks, dtype=torch.int64, device=w.q.device)
    return (np.array(ind, dtype=np.int32), np.array(idx, dtype=np.int32),
            w.last_page_len[list(rows)].astype(np.int32), qo, t)


CASES = [
    # (seed, head_dim, Hq, Hk, page_size, window)
    (600, 128, 32, 8, 16, -1),    # one launch
    (601, 64, 16, 16, 32, 300),   # one launch, group 1, window
    (602, 128, 64, 8, 16, -1),    # one launch, group 8
    (603, 64, 8, 2, 4, -1),       # two launches (page_size < 16)
    (604, 128, 16, 4, 8, 50),     # two launches, window
]


def _random_mixed_shapes(n=8, seed=4343):
    """Seeded mixed shapes: head dims, decode-supported groups, page sizes on
    both sides of the one-launch threshold (16), windows."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        hk = int(rng.choice([1, 2, 4]))
        ps = int(rng.choice([1, 4, 8, 16, 32, 64]))
        wl = int(rng.choice([-1, -1, 0, 25, 400]))
        out.append((620 + k, D, g * hk, hk, ps, wl))
    return out


CASES += _random_mixed_shapes()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-D{c[1]}-g{c[2]//c[3]}-ps{c[4]}-w{c[5]}")
def test_mixed_equals_decode_plus_prefill(pkv, gpu, case):
    seed, D, hq, hk, ps, wl = case
    say(f"case mixed seed={seed} D={D} Hq={hq} Hk={hk} ps={ps} window={wl}")
    rng = np.random.default_rng(seed)
    B = 14
    kv = rng.integers(1, 900, size=B)
    ql = np.ones(B, dtype=np.int64)
    for r in rng.choice(B, size=4, replace=False):
        ql[r] = int(rng.integers(2, min(int(kv[r]), 300) + 1)) if kv[r] >= 2 else 1
    w = synth.from_lengths(f"mixed{seed}", "mixed", kv, ql, num_qo_heads=hq, num_kv_heads=hk,
                           head_dim=D, page_size=ps, window_left=wl, seed=seed, device=gpu,
                           stale="nan", max_prefill_rows=4)
    # split rows so that merges run, in the mixed plan and in the decode plan alike
    kw = dict(num_cus=16, decode_waves_per_cu=8, decode_min_chunk_pages=1)
    out, lse, plan, _ = gpu_run(pkv, w, **kw)
    dec = [r for r in range(B) if ql[r] == 1]
    pre = [r for r in range(B) if ql[r] >= 2]
    assert dec and pre and plan.info()["decode_rows"] == len(dec)
    for kind, rows in (("decode", dec), ("prefill", pre)):
        ind, idx, lpl, qo, toks = _sub(w, rows, kind)
        p = pkv.plan_params(kind, num_qo_heads=hq, num_kv_heads=hk, head_dim=D, page_size=ps,
                            max_pages=w.max_pages, window_left=wl, **kw)
        sp = pkv.plan_create(p, None if kind == "decode" else qo, ind, idx, lpl)
        ws = torch.empty(sp.ws_bytes, dtype=torch.uint8, device=gpu)
        pkv.plan_upload(sp, ws)
        q = w.q[toks].contiguous()
        o2 = torch.full_like(q, float("nan"))
        l2 = torch.full((q.shape[0], hq), float("nan"), dtype=torch.float32, device=gpu)
        pkv.run(sp, q, w.cache, o2, ws, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(out[toks].view(torch.int16), o2.view(torch.int16)), f"{kind} rows: out"
        assert torch.equal(lse[toks].view(torch.int32), l2.view(torch.int32)), f"{kind} rows: lse"
    ref_o, ref_l = oracle.attention(w.q.cpu(), w.cache.cpu(), ps, w.kv_indptr, w.kv_indices,
                                    w.last_page_len, num_qo_heads=hq, num_kv_heads=hk,
                                    qo_indptr=w.qo_indptr, causal=True, window_left=wl)
    compare(out, lse, ref_o, ref_l, f"mixed s{seed}")
