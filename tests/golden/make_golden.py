"""Write tests/golden/tiny_decode.json: the oracle's output for the tiny decode
workload (4 requests, 4 query heads over 2 KV heads, head_dim 64, page size 16,
kv_len uniform in [1, 100], seed 1001).

Calls only oracle/ and synth/.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    w = synth.make_workload("tiny_decode")
    out, lse = oracle.attention(w.q, w.cache, w.page_size, w.kv_indptr, w.kv_indices,
                                w.last_page_len, num_qo_heads=w.num_qo_heads,
                                num_kv_heads=w.num_kv_heads)
    slots = oracle.write_slots(w.page_size, w.kv_indptr, w.kv_indices, w.last_page_len)
    doc = {
        "what": "oracle output for the tiny decode workload (seed 1001)",
        "kv_len": [int(x) for x in w.kv_len],
        "kv_indices": [int(x) for x in w.kv_indices],
        "last_page_len": [int(x) for x in w.last_page_len],
        "write_slots": [int(x) for x in slots],
        "out": np.round(out, 15).tolist(),
        "lse": np.round(lse, 15).tolist(),
    }
    with open(os.path.join(os.path.dirname(__file__), "tiny_decode.json"), "w") as f:
        json.dump(doc, f)


if __name__ == "__main__":
    main()
