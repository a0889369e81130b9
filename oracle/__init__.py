"""CPU oracle for batched attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only tests/, the smoke check in __graft_entry__ and the benchmark's CPU
baseline leg may use it.  It shares no code with the HIP library.

Everything here is plain numpy in float64, written from the definition of the
operation rather than from any kernel design:

  * the page table (mstar.engine.resources.kv.plan: PagedIndptrs and
    SequenceView.last_page_len) decoded into per-row token counts;
  * each row's logical K/V gathered page by page out of a layer slice laid out
    [max_pages, 2, page_size, num_kv_heads, head_dim]
    (mstar.engine.resources.attn.wrappers: module docstring, the run methods);
  * softmax(q k^T / sqrt(head_dim)) v with a causal mask aligned to the end of
    the row's KV (a [cached prefix | fresh tokens] sequence,
    mstar.engine.resources.attn.dense: DenseAttentionManager) and the
    window_left bound (FlashInferPrefillWrapper.plan);
  * the write location of each appended token (FlashInferDecodeWrapper.plan;
    kv.plan: KVPlanOutput decode_pages / decode_offsets);
  * the mixed step's token permutation (FlashInferMixedWrapper);
  * the merge of split-KV partials by log-sum-exp
    (mstar.engine.resources.attn.workspace, module docstring).

Parity status: every function is pinned by tests/test_oracle_pins.py except the
two conventions no page fixes (index 0 of the "2" axis is K, and query head h
reads KV head h // (num_qo_heads // num_kv_heads)): those are "parity unpinned".
"""
from .reference import *  # noqa: F401,F403
from .plan_check import *  # noqa: F401,F403
