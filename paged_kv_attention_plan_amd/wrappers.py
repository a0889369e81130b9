"""Decode, prefill and mixed-step wrappers over the C ABI.

Shaped like the wrappers of the mstar attn.wrappers page
(FlashInferDecodeWrapper, FlashInferPrefillWrapper, FlashInferMixedWrapper):
construct with a workspace and the head/page geometry, call plan() with host
index arrays once per step, then run(q, kv_cache_layer) per layer.  KV writes
are a separate call, append_kv(), made before run() (attn.dense,
requires_kv_write).

The workspace is a torch uint8 device tensor.  A plan that needs more than it
holds grows it (a new tensor of the exact size), as the workspace page's
Workspace.plan does; once seal() is called the address is frozen and an
overflow raises with the bytes the plan asked for.

DenseWrapper is the dense [frozen prefix | fresh tokens] path of the attn.dense
page (DenseAttentionManager, DensePlan): plan(cu_q, cu_k) once per step,
gather() builds the contiguous K/V (the prefixes once, the fresh rows every
step), run(q, k, v) per layer; the fresh K/V never reach the pages.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import pkv

__all__ = ["DecodeWrapper", "PrefillWrapper", "MixedWrapper", "DenseWrapper", "WorkspaceTooSmall"]

_INT32_MAX = 2 ** 31 - 1


class WorkspaceTooSmall(RuntimeError):
    pass


class _Wrapper:
    _kind = "decode"

    def __init__(self, workspace_buffer: Optional[torch.Tensor], num_qo_heads: int,
                 num_kv_heads: int, head_dim: int, page_size: int, max_num_pages=None,
                 device="cuda", max_prefill_rows: int = 0, num_cus: int = 0):
        self.num_qo_heads = num_qo_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.page_size = page_size
        self.max_num_pages = max_num_pages
        self.device = torch.device(device)
        self.max_prefill_rows = max_prefill_rows
        self.num_cus = num_cus
        if workspace_buffer is None:
            workspace_buffer = torch.empty(0, dtype=torch.uint8, device=self.device)
        self.workspace = workspace_buffer
        self.sealed = False
        self._plan: Optional[pkv.Plan] = None
        self._planned = False  # the handle's plan is the one in the workspace
        self._key = None
        self._max_page_id = -1

    def seal(self):
        """Freeze the workspace address: later plans that do not fit raise."""
        self.sealed = True

    def _do_plan(self, qo_indptr, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
                 kv_lens, causal, window_left):
        max_pages = self.max_num_pages if self.max_num_pages is not None else _INT32_MAX
        key = (bool(causal), int(window_left))
        if self._plan is None or key != self._key:
            params = pkv.plan_params(self._kind, num_qo_heads=self.num_qo_heads,
                                     num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                                     page_size=self.page_size, max_pages=max_pages, causal=causal,
                                     window_left=window_left,
                                     max_prefill_rows=self.max_prefill_rows, num_cus=self.num_cus)
            self._plan = pkv.plan_create(params, qo_indptr, paged_kv_indptr, paged_kv_indices,
                                         paged_kv_last_page_len, kv_lens)
            self._key = key
        else:
            pkv.plan_update(self._plan, qo_indptr, paged_kv_indptr, paged_kv_indices,
                            paged_kv_last_page_len, kv_lens)
        need = self._plan.ws_bytes
        have = self.workspace.numel() * self.workspace.element_size()
        if have < need:
            if self.sealed:
                # the handle now holds a plan the workspace cannot take: no run
                # until a plan() succeeds
                self._planned = False
                raise WorkspaceTooSmall(
                    f"plan needs {need} workspace bytes; the sealed workspace holds {have}")
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        idx = np.asarray(paged_kv_indices.cpu() if hasattr(paged_kv_indices, "cpu") else paged_kv_indices)
        self._max_page_id = int(idx.max()) if idx.size else -1
        pkv.plan_upload(self._plan, self.workspace)
        self._planned = True

    @property
    def plan_handle(self) -> pkv.Plan:
        if not self._planned:
            raise RuntimeError("no successful plan(): call plan() before run() / append_kv()")
        return self._plan

    def _check_cache(self, kv_cache_layer):
        shp = tuple(kv_cache_layer.shape)
        if len(shp) != 5 or shp[1:] != (2, self.page_size, self.num_kv_heads, self.head_dim):
            raise ValueError(f"kv_cache_layer must be [max_pages, 2, {self.page_size}, "
                             f"{self.num_kv_heads}, {self.head_dim}], got {shp}")
        if self._max_page_id >= shp[0]:
            raise ValueError(f"page id {self._max_page_id} outside a cache of {shp[0]} pages")

    def run(self, q: torch.Tensor, kv_cache_layer: torch.Tensor, return_lse: bool = False,
            out: Optional[torch.Tensor] = None):
        plan = self.plan_handle
        self._check_cache(kv_cache_layer)
        if q.dim() != 3 or q.shape[1:] != (self.num_qo_heads, self.head_dim):
            raise ValueError(f"q must be [tokens, {self.num_qo_heads}, {self.head_dim}]")
        if q.shape[0] != plan.info()["total_q"]:
            raise ValueError("q has a different token count than the plan")
        if out is None:
            out = torch.empty_like(q)
        lse = (torch.empty(q.shape[0], self.num_qo_heads, dtype=torch.float32, device=q.device)
               if return_lse else None)
        pkv.run(plan, q, kv_cache_layer, out, self.workspace, lse=lse)
        return (out, lse) if return_lse else out

    def append_kv(self, k_new: torch.Tensor, v_new: torch.Tensor, kv_cache_layer: torch.Tensor):
        """Store this step's K/V at the planned write slots (before run)."""
        self._check_cache(kv_cache_layer)
        shape = (self.plan_handle.info()["total_q"], self.num_kv_heads, self.head_dim)
        if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
            raise ValueError(f"k_new and v_new must be {shape}")
        pkv.append_kv(self.plan_handle, k_new, v_new, kv_cache_layer, self.workspace)


class DecodeWrapper(_Wrapper):
    """Batched decode: one query token per request (FlashInferDecodeWrapper)."""
    _kind = "decode"

    def plan(self, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
             dtype=torch.bfloat16, kv_lens=None, window_left=-1):
        if dtype != torch.bfloat16:
            raise pkv.PkvError(pkv.E_UNSUPPORTED, "only bf16 is supported")
        self._do_plan(None, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len, kv_lens,
                      True, window_left)


class PrefillWrapper(_Wrapper):
    """Batched ragged prefill over a paged cache (FlashInferPrefillWrapper)."""
    _kind = "prefill"

    def plan(self, qo_indptr, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
             causal=True, dtype=torch.bfloat16, kv_lens=None, window_left=-1):
        if dtype != torch.bfloat16:
            raise pkv.PkvError(pkv.E_UNSUPPORTED, "only bf16 is supported")
        self._do_plan(qo_indptr, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
                      kv_lens, causal, window_left)


class MixedWrapper(_Wrapper):
    """One-token rows on a decode sub-plan, prompt rows (at most
    max_prefill_rows) on a prefill sub-plan, one output tensor
    (FlashInferMixedWrapper).  Both sub-plans share one plan handle and one
    workspace; the prompt tokens' "move to the front" is folded into the
    prefill kernel's addressing instead of a copy of q."""
    _kind = "mixed"

    def plan(self, qo_indptr, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
             causal=True, dtype=torch.bfloat16, kv_lens=None, window_left=-1):
        if dtype != torch.bfloat16:
            raise pkv.PkvError(pkv.E_UNSUPPORTED, "only bf16 is supported")
        self._do_plan(qo_indptr, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
                      kv_lens, causal, window_left)


class DenseWrapper:
    """Dense varlen attention over contiguous [prefix | fresh] K/V
    (attn.dense DenseAttentionManager / DensePlan).  Row r's queries are
    q[cu_q[r]:cu_q[r+1]] and its keys k/v[cu_k[r]:cu_k[r+1]], the last
    cu_q[r+1] - cu_q[r] of them fresh."""

    def __init__(self, workspace_buffer: Optional[torch.Tensor], num_qo_heads: int,
                 num_kv_heads: int, head_dim: int, page_size: int, max_num_pages=None,
                 device="cuda", num_cus: int = 0):
        self.num_qo_heads, self.num_kv_heads, self.head_dim = num_qo_heads, num_kv_heads, head_dim
        self.page_size = page_size
        self.max_num_pages = max_num_pages
        self.device = torch.device(device)
        self.num_cus = num_cus
        if workspace_buffer is None:
            workspace_buffer = torch.empty(0, dtype=torch.uint8, device=self.device)
        self.workspace = workspace_buffer
        self.sealed = False
        self._plan: Optional[pkv.Plan] = None
        self._planned = False
        self._key = None

    def seal(self):
        """Freeze the workspace address: later plans that do not fit raise."""
        self.sealed = True

    def plan(self, cu_q, cu_k, paged_kv_indptr=None, paged_kv_indices=None, causal=True,
             dtype=torch.bfloat16, window_left=-1):
        """Plan a step.  The page table (each row's pages, holding at least its
        prefix) is needed only to gather prefixes out of the pages."""
        if dtype != torch.bfloat16:
            raise pkv.PkvError(pkv.E_UNSUPPORTED, "only bf16 is supported")
        key = (bool(causal), int(window_left))
        if self._plan is None or key != self._key:
            max_pages = self.max_num_pages if self.max_num_pages is not None else _INT32_MAX
            params = pkv.plan_params("dense", num_qo_heads=self.num_qo_heads,
                                     num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                                     page_size=self.page_size, max_pages=max_pages, causal=causal,
                                     window_left=window_left, num_cus=self.num_cus)
            self._plan = pkv.dense_plan_create(params, cu_q, cu_k, paged_kv_indptr,
                                               paged_kv_indices)
            self._key = key
        else:
            pkv.dense_plan_update(self._plan, cu_q, cu_k, paged_kv_indptr, paged_kv_indices)
        need = self._plan.ws_bytes
        have = self.workspace.numel() * self.workspace.element_size()
        if have < need:
            if self.sealed:
                self._planned = False
                raise WorkspaceTooSmall(
                    f"plan needs {need} workspace bytes; the sealed workspace holds {have}")
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        pkv.plan_upload(self._plan, self.workspace)
        self._planned = True

    @property
    def plan_handle(self) -> pkv.Plan:
        if not self._planned:
            raise RuntimeError("no successful plan(): call plan() before gather() / run()")
        return self._plan

    def gather(self, kv_cache_layer, k_fresh, v_fresh, k_out=None, v_out=None,
               with_prefix=True):
        """Contiguous K and V [cu_k[-1], Hk, D]: each row's prefix from the
        pages (with_prefix) followed by its fresh K/V.  Pass the previous
        k_out / v_out with with_prefix=False to refresh only the fresh rows."""
        info = self.plan_handle.info()
        shape = (info["total_k"], self.num_kv_heads, self.head_dim)
        if k_out is None:
            k_out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        if v_out is None:
            v_out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        pkv.dense_gather(self.plan_handle, kv_cache_layer, k_fresh, v_fresh, k_out, v_out,
                         self.workspace, with_prefix=with_prefix)
        return k_out, v_out

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, return_lse: bool = False,
            out: Optional[torch.Tensor] = None):
        if out is None:
            out = torch.empty_like(q)
        lse = (torch.empty(q.shape[0], self.num_qo_heads, dtype=torch.float32, device=q.device)
               if return_lse else None)
        pkv.dense_run(self.plan_handle, q, k, v, out, self.workspace, lse=lse)
        return (out, lse) if return_lse else out
