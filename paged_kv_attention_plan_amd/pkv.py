"""ctypes binding of libpkv.so (include/pkv.h), one Python function per C call.

Argument marshalling only: host index arrays become int32 pointers, torch
device tensors become raw device pointers, the stream is the current HIP
stream.  Every step of the path runs in the library.  There is no fallback:
if libpkv.so is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

# ---- status codes and enums (pkv.h) ----
OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_CAPACITY, E_CONFLICT, E_DEVICE, E_STATE = range(8)
KIND_DECODE, KIND_PREFILL, KIND_MIXED, KIND_DENSE = 0, 1, 2, 3
DTYPE_BF16 = 0
_KINDS = {"decode": KIND_DECODE, "prefill": KIND_PREFILL, "mixed": KIND_MIXED, "dense": KIND_DENSE}

STATUS_NAMES = {OK: "PKV_OK", E_INVALID: "PKV_E_INVALID", E_UNSUPPORTED: "PKV_E_UNSUPPORTED",
                E_WORKSPACE: "PKV_E_WORKSPACE", E_CAPACITY: "PKV_E_CAPACITY",
                E_CONFLICT: "PKV_E_CONFLICT", E_DEVICE: "PKV_E_DEVICE", E_STATE: "PKV_E_STATE"}


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class PlanParams(C.Structure):
    _fields_ = [("kind", C.c_int32), ("num_qo_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("page_size", C.c_int32), ("causal", C.c_int32),
                ("window_left", C.c_int32), ("dtype", C.c_int32), ("max_prefill_rows", C.c_int32),
                ("num_cus", C.c_int32), ("max_pages", C.c_int64),
                ("decode_waves_per_cu", C.c_int32), ("decode_min_chunk_pages", C.c_int32),
                ("static_max_batch", C.c_int32), ("static_max_tokens", C.c_int32),
                ("static_max_page_entries", C.c_int64)]


DECODE_TILE = np.dtype([("row", "<i4"), ("kv_head", "<i4"), ("kv_start", "<i4"), ("kv_end", "<i4"),
                        ("page_base", "<i4"), ("q_index", "<i4"), ("out_slot", "<i4"),
                        ("kv_len", "<i4")])
MERGE_ENTRY = np.dtype([("q_index", "<i4"), ("kv_head", "<i4"), ("slot_base", "<i4"),
                        ("n_chunks", "<i4")])
PREFILL_TILE = np.dtype([("row", "<i4"), ("kv_head", "<i4"), ("q_start", "<i4"),
                         ("q_count", "<i4"), ("kv_lo", "<i4"), ("kv_hi", "<i4"),
                         ("page_base", "<i4"), ("q_base", "<i4"), ("kv_len", "<i4"),
                         ("q_len", "<i4"), ("pad0", "<i4"), ("pad1", "<i4")])


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run "
                           "`python -m paged_kv_attention_plan_amd.build` (ROCm hipcc, gfx950)")
    lib = C.CDLL(LIB_PATH)
    P = C.POINTER
    i32p = P(C.c_int32)
    sig = {
        "pkv_plan_params_init": (None, [P(PlanParams)]),
        "pkv_plan_create": (C.c_int, [P(PlanParams), C.c_int32, i32p, i32p, i32p, i32p, i32p,
                                      P(C.c_void_p), P(C.c_size_t)]),
        "pkv_plan_update": (C.c_int, [C.c_void_p, C.c_int32, i32p, i32p, i32p, i32p, i32p,
                                      P(C.c_size_t)]),
        "pkv_plan_destroy": (None, [C.c_void_p]),
        "pkv_plan_decode_tiles": (C.c_int, [C.c_void_p, P(C.c_void_p), P(C.c_int32)]),
        "pkv_plan_prefill_tiles": (C.c_int, [C.c_void_p, P(C.c_void_p), P(C.c_int32)]),
        "pkv_plan_merges": (C.c_int, [C.c_void_p, P(C.c_void_p), P(C.c_int32)]),
        "pkv_plan_write_slots": (C.c_int, [C.c_void_p, P(C.c_void_p), P(C.c_int32)]),
        "pkv_plan_permutation": (C.c_int, [C.c_void_p, P(C.c_void_p), P(C.c_int32)]),
        "pkv_plan_info": (C.c_int, [C.c_void_p, P(C.c_int64)]),
        "pkv_plan_upload": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
        "pkv_plan_upload_stats": (C.c_int, [C.c_void_p, P(C.c_int64)]),
        "pkv_run": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_size_t, C.c_void_p]),
        "pkv_append_kv": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_size_t, C.c_void_p]),
        "pkv_run_append": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
        "pkv_plan_metadata": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t]),
        "pkv_run_noalloc": (C.c_int, [C.c_void_p] * 6),
        "pkv_noalloc_capacity": (C.c_size_t, []),
        "pkv_context_only_views": (C.c_int, [C.c_int32, C.c_int32] + [P(C.c_int32)] * 9),
        "pkv_dense_plan_create": (C.c_int, [C.c_void_p, C.c_int32] + [P(C.c_int32)] * 4
                                  + [P(C.c_void_p), P(C.c_size_t)]),
        "pkv_dense_plan_update": (C.c_int, [C.c_void_p, C.c_int32] + [P(C.c_int32)] * 4
                                  + [P(C.c_size_t)]),
        "pkv_dense_gather": (C.c_int, [C.c_void_p] * 6 + [C.c_int32, C.c_void_p, C.c_size_t,
                                                         C.c_void_p]),
        "pkv_dense_run": (C.c_int, [C.c_void_p] * 5 + [C.c_void_p, C.c_void_p, C.c_size_t,
                                                      C.c_void_p]),
        "pkv_timing_enable": (C.c_int, [C.c_void_p, C.c_int32]),
        "pkv_timing_read": (C.c_int, [C.c_void_p, P(C.c_double), P(C.c_int64)]),
        "pkv_last_error": (C.c_char_p, []),
        "pkv_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("pkv_plan_params_init", "pkv_plan_create", "pkv_plan_update", "pkv_plan_destroy",
            "pkv_plan_decode_tiles", "pkv_plan_prefill_tiles", "pkv_plan_merges",
            "pkv_plan_write_slots", "pkv_plan_permutation", "pkv_plan_info", "pkv_plan_metadata",
            "pkv_plan_upload", "pkv_plan_upload_stats",
            "pkv_run", "pkv_append_kv", "pkv_run_append", "pkv_run_noalloc", "pkv_noalloc_capacity",
            "pkv_context_only_views",
            "pkv_dense_plan_create", "pkv_dense_plan_update", "pkv_dense_gather", "pkv_dense_run",
            "pkv_timing_enable", "pkv_timing_read",
            "pkv_last_error", "pkv_version")


def _check(status: int):
    if status != OK:
        raise PkvError(status, _lib.pkv_last_error().decode())


def _i32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (host)
        if a.device.type != "cpu":
            raise ValueError("plan inputs must be host arrays (pass CPU tensors or numpy arrays)")
        a = a.detach().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(C.POINTER(C.c_int32))


def version() -> str:
    return _lib.pkv_version().decode()


def plan_params(kind="decode", *, num_qo_heads, num_kv_heads, head_dim, page_size, max_pages,
                causal=True, window_left=-1, max_prefill_rows=0, num_cus=0,
                decode_waves_per_cu=0, decode_min_chunk_pages=0, static_max_batch=0,
                static_max_tokens=0, static_max_page_entries=0) -> PlanParams:
    p = PlanParams()
    _lib.pkv_plan_params_init(C.byref(p))
    p.kind = _KINDS[kind] if isinstance(kind, str) else int(kind)
    p.num_qo_heads, p.num_kv_heads, p.head_dim, p.page_size = num_qo_heads, num_kv_heads, head_dim, page_size
    p.causal, p.window_left, p.dtype = int(bool(causal)), int(window_left), DTYPE_BF16
    p.max_prefill_rows, p.num_cus, p.max_pages = int(max_prefill_rows), int(num_cus), int(max_pages)
    p.decode_waves_per_cu, p.decode_min_chunk_pages = int(decode_waves_per_cu), int(decode_min_chunk_pages)
    p.static_max_batch, p.static_max_tokens = int(static_max_batch), int(static_max_tokens)
    p.static_max_page_entries = int(static_max_page_entries)
    return p


class Plan:
    """Owner of a pkv_plan handle."""

    def __init__(self, handle, ws_bytes: int, params: PlanParams, max_page_id: int = -1):
        self._h = handle
        self.ws_bytes = ws_bytes
        self.params = params
        self.max_page_id = max_page_id

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.pkv_plan_destroy(h)

    def _arr(self, fn, dtype):
        ptr, n = C.c_void_p(), C.c_int32()
        _check(fn(self._h, C.byref(ptr), C.byref(n)))
        if n.value == 0:
            return np.zeros(0, dtype=dtype)
        buf = (C.c_char * (n.value * dtype.itemsize)).from_address(ptr.value)
        return np.frombuffer(buf, dtype=dtype).copy()

    def decode_tiles(self):
        return self._arr(_lib.pkv_plan_decode_tiles, DECODE_TILE)

    def prefill_tiles(self):
        return self._arr(_lib.pkv_plan_prefill_tiles, PREFILL_TILE)

    def merges(self):
        return self._arr(_lib.pkv_plan_merges, MERGE_ENTRY)

    def write_slots(self):
        return self._arr(_lib.pkv_plan_write_slots, np.dtype("<i8"))

    def permutation(self):
        return self._arr(_lib.pkv_plan_permutation, np.dtype("<i4"))

    def metadata(self) -> np.ndarray:
        """pkv_plan_metadata: the bytes the upload puts at the head of the workspace."""
        n = self.info()["meta_bytes"]
        buf = np.zeros(n, dtype=np.uint8)
        _check(_lib.pkv_plan_metadata(self._h, buf.ctypes.data_as(C.c_void_p), n))
        return buf

    def upload_stats(self) -> dict:
        """pkv_plan_upload_stats: uploads launched, uploads that waited for their
        staging buffer's previous reader, and the nanoseconds spent waiting."""
        v = (C.c_int64 * 3)()
        _check(_lib.pkv_plan_upload_stats(self._h, v))
        return {"uploads": int(v[0]), "waits": int(v[1]), "wait_ns": int(v[2])}

    def info(self) -> dict:
        v = (C.c_int64 * 18)()
        _check(_lib.pkv_plan_info(self._h, v))
        keys = ["total_q", "batch", "decode_rows", "prompt_rows", "worker_pages", "partial_slots",
                "meta_bytes", "workspace_bytes", "num_cus", "total_k", "off_dense_rows",
                "off_decode_rows", "off_decode_pieces", "off_merges", "off_prefill_tiles",
                "off_indices", "off_decode_work", "decode_workers"]
        return {k: int(v[i]) for i, k in enumerate(keys)}


def plan_create(params: PlanParams, qo_indptr, paged_kv_indptr, paged_kv_indices,
                paged_kv_last_page_len, kv_lens=None) -> Plan:
    """pkv_plan_create: validate the page table and build a plan (host only)."""
    qo, ind, idx, lpl, kvl = map(_i32, (qo_indptr, paged_kv_indptr, paged_kv_indices,
                                        paged_kv_last_page_len, kv_lens))
    batch = len(lpl)
    h, ws = C.c_void_p(), C.c_size_t()
    _check(_lib.pkv_plan_create(C.byref(params), batch, _ptr(qo), _ptr(ind), _ptr(idx), _ptr(lpl),
                                _ptr(kvl), C.byref(h), C.byref(ws)))
    return Plan(h.value, ws.value, params, int(idx.max()) if idx.size else -1)


def plan_update(plan: Plan, qo_indptr, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
                kv_lens=None) -> int:
    """pkv_plan_update: re-plan the same handle for a new step; returns workspace bytes."""
    qo, ind, idx, lpl, kvl = map(_i32, (qo_indptr, paged_kv_indptr, paged_kv_indices,
                                        paged_kv_last_page_len, kv_lens))
    ws = C.c_size_t()
    _check(_lib.pkv_plan_update(plan.handle, len(lpl), _ptr(qo), _ptr(ind), _ptr(idx), _ptr(lpl),
                                _ptr(kvl), C.byref(ws)))
    plan.ws_bytes = ws.value
    plan.max_page_id = int(idx.max()) if idx.size else -1
    return ws.value


def _stream(stream):
    """A hipStream_t for the C calls: a torch stream, a raw handle, or (None)
    torch's current stream."""
    if stream is not None:
        return C.c_void_p(int(getattr(stream, "cuda_stream", stream)))
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return C.c_void_p(t.data_ptr())


def plan_upload(plan: Plan, workspace, stream=None):
    """pkv_plan_upload: async copy of the plan metadata into the workspace head."""
    _check(_lib.pkv_plan_upload(plan.handle, _dev(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


def _check_sizes(plan: Plan, kv_cache_layer, **tensors):
    """The C ABI takes raw pointers; make sure the tensors hold what the plan
    will touch before handing them over."""
    pp = plan.params
    # graph-static plans take buffers sized for their capacity, whatever the step holds
    T = pp.static_max_tokens if pp.static_max_batch > 0 else plan.info()["total_q"]
    want = {"q": T * pp.num_qo_heads * pp.head_dim, "out": T * pp.num_qo_heads * pp.head_dim,
            "lse": T * pp.num_qo_heads, "k_new": T * pp.num_kv_heads * pp.head_dim,
            "v_new": T * pp.num_kv_heads * pp.head_dim}
    for name, t in tensors.items():
        if t is not None and t.numel() != want[name]:
            raise ValueError(f"{name} has {t.numel()} elements; the plan needs {want[name]}")
    page = 2 * pp.page_size * pp.num_kv_heads * pp.head_dim
    if kv_cache_layer.numel() % page != 0:
        raise ValueError("kv_cache_layer is not a whole number of pages")
    if plan.max_page_id >= kv_cache_layer.numel() // page:
        raise ValueError(f"the plan reads page {plan.max_page_id}; kv_cache_layer holds "
                         f"{kv_cache_layer.numel() // page} pages")


def run(plan: Plan, q, kv_cache_layer, out, workspace, lse=None, stream=None):
    """pkv_run: attention for every planned query, written into out (and lse)."""
    import torch
    _check_sizes(plan, kv_cache_layer, q=q, out=out, lse=lse)
    _check(_lib.pkv_run(plan.handle, _dev(q, "q", torch.bfloat16),
                        _dev(kv_cache_layer, "kv_cache_layer", torch.bfloat16),
                        _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32),
                        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                        _stream(stream)))


def run_noalloc(plan: Plan, q, kv_cache_layer, out, lse=None, stream=None):
    """pkv_run_noalloc: upload + run with the library's static per-GPU workspace
    (no allocation; the plan must have been uploaded once with plan_upload so
    that its staging buffers hold its metadata)."""
    import torch
    _check_sizes(plan, kv_cache_layer, q=q, out=out, lse=lse)
    _check(_lib.pkv_run_noalloc(plan.handle, _dev(q, "q", torch.bfloat16),
                                _dev(kv_cache_layer, "kv_cache_layer", torch.bfloat16),
                                _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32),
                                _stream(stream)))


def noalloc_capacity() -> int:
    """pkv_noalloc_capacity: bytes of the static workspace of run_noalloc."""
    return int(_lib.pkv_noalloc_capacity())


def run_append(plan: Plan, q, k_new, v_new, kv_cache_layer, out, workspace, lse=None, stream=None):
    """pkv_run_append: store this step's K/V, then run attention (append_kv
    followed by run on one stream)."""
    import torch
    _check_sizes(plan, kv_cache_layer, q=q, out=out, lse=lse, k_new=k_new, v_new=v_new)
    _check(_lib.pkv_run_append(plan.handle, _dev(q, "q", torch.bfloat16),
                               _dev(k_new, "k_new", torch.bfloat16),
                               _dev(v_new, "v_new", torch.bfloat16),
                               _dev(kv_cache_layer, "kv_cache_layer", torch.bfloat16),
                               _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32),
                               _dev(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(stream)))


def append_kv(plan: Plan, k_new, v_new, kv_cache_layer, workspace, stream=None):
    """pkv_append_kv: store this step's K/V at the planned write slots."""
    import torch
    _check_sizes(plan, kv_cache_layer, k_new=k_new, v_new=v_new)
    _check(_lib.pkv_append_kv(plan.handle, _dev(k_new, "k_new", torch.bfloat16),
                              _dev(v_new, "v_new", torch.bfloat16),
                              _dev(kv_cache_layer, "kv_cache_layer", torch.bfloat16),
                              _dev(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream)))


TIMING_KINDS = ("append", "decode", "merge", "prefill")


def dense_plan_create(params: PlanParams, cu_q, cu_k, paged_kv_indptr=None,
                      paged_kv_indices=None) -> Plan:
    """pkv_dense_plan_create: rows of contiguous [prefix | fresh] K/V at cu_k
    offsets, queries at cu_q offsets; the optional page table lets
    dense_gather copy each row's prefix out of the pages (host only)."""
    cq, ck, ind, idx = map(_i32, (cu_q, cu_k, paged_kv_indptr, paged_kv_indices))
    batch = len(cq) - 1
    if batch < 0 or len(ck) != batch + 1:
        raise PkvError(1, "cu_q and cu_k need batch + 1 entries")
    h, ws = C.c_void_p(), C.c_size_t()
    _check(_lib.pkv_dense_plan_create(C.byref(params), batch, _ptr(cq), _ptr(ck), _ptr(ind),
                                      _ptr(idx), C.byref(h), C.byref(ws)))
    return Plan(h.value, ws.value, params, int(idx.max()) if idx is not None and idx.size else -1)


def dense_plan_update(plan: Plan, cu_q, cu_k, paged_kv_indptr=None, paged_kv_indices=None) -> int:
    """pkv_dense_plan_update: re-plan a dense handle; returns workspace bytes."""
    cq, ck, ind, idx = map(_i32, (cu_q, cu_k, paged_kv_indptr, paged_kv_indices))
    batch = len(cq) - 1
    if batch < 0 or len(ck) != batch + 1:
        raise PkvError(1, "cu_q and cu_k need batch + 1 entries")
    ws = C.c_size_t()
    _check(_lib.pkv_dense_plan_update(plan.handle, batch, _ptr(cq), _ptr(ck), _ptr(ind), _ptr(idx),
                                      C.byref(ws)))
    plan.ws_bytes = ws.value
    plan.max_page_id = int(idx.max()) if idx is not None and idx.size else -1
    return ws.value


def _check_dense_sizes(plan: Plan, **tensors):
    pp = plan.params
    info = plan.info()
    T, K = info["total_q"], info["total_k"]
    row_q, row_k = pp.num_qo_heads * pp.head_dim, pp.num_kv_heads * pp.head_dim
    want = {"q": T * row_q, "out": T * row_q, "lse": T * pp.num_qo_heads, "k": K * row_k,
            "v": K * row_k, "k_fresh": T * row_k, "v_fresh": T * row_k, "k_out": K * row_k,
            "v_out": K * row_k}
    for name, t in tensors.items():
        if t is not None and t.numel() != want[name]:
            raise ValueError(f"{name} has {t.numel()} elements; the plan needs {want[name]}")


def dense_gather(plan: Plan, kv_cache_layer, k_fresh, v_fresh, k_out, v_out, workspace,
                 with_prefix=True, stream=None):
    """pkv_dense_gather: fill k_out / v_out with each row's prefix (from the
    pages, if with_prefix) and its fresh K/V."""
    import torch
    _check_dense_sizes(plan, k_fresh=k_fresh, v_fresh=v_fresh, k_out=k_out, v_out=v_out)
    if with_prefix:
        pp = plan.params
        page = 2 * pp.page_size * pp.num_kv_heads * pp.head_dim
        if kv_cache_layer is None or plan.max_page_id >= kv_cache_layer.numel() // page:
            raise ValueError("kv_cache_layer does not hold the plan's pages")
    _check(_lib.pkv_dense_gather(plan.handle, _dev(kv_cache_layer, "kv_cache_layer", torch.bfloat16),
                                 _dev(k_fresh, "k_fresh", torch.bfloat16),
                                 _dev(v_fresh, "v_fresh", torch.bfloat16),
                                 _dev(k_out, "k_out", torch.bfloat16),
                                 _dev(v_out, "v_out", torch.bfloat16), int(bool(with_prefix)),
                                 _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def dense_run(plan: Plan, q, k, v, out, workspace, lse=None, stream=None):
    """pkv_dense_run: attention over contiguous [prefix | fresh] K/V."""
    import torch
    _check_dense_sizes(plan, q=q, k=k, v=v, out=out, lse=lse)
    _check(_lib.pkv_dense_run(plan.handle, _dev(q, "q", torch.bfloat16),
                              _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16),
                              _dev(out, "out", torch.bfloat16), _dev(lse, "lse", torch.float32),
                              _dev(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream)))


def context_only_views(page_size, paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
                       to_compute, query_spans):
    """pkv_context_only_views: the page table without the step's appended
    tokens.  Returns (paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
    qo_indptr) as int32 arrays; plan them with causal=False."""
    ind, idx, lpl, tc, qs = map(_i32, (paged_kv_indptr, paged_kv_indices, paged_kv_last_page_len,
                                       to_compute, query_spans))
    batch = len(lpl)
    o_ind = np.zeros(batch + 1, dtype=np.int32)
    o_idx = np.zeros(max(len(idx), 1), dtype=np.int32)
    o_lpl = np.zeros(max(batch, 1), dtype=np.int32)
    o_qo = np.zeros(batch + 1, dtype=np.int32)
    if len(ind) != batch + 1 or len(tc) != batch or len(qs) != batch:
        raise PkvError(1, "paged_kv_indptr needs batch + 1 entries and to_compute / query_spans "
                          "batch entries")
    _check(_lib.pkv_context_only_views(batch, int(page_size), _ptr(ind), _ptr(idx), _ptr(lpl),
                                       _ptr(tc), _ptr(qs), _ptr(o_ind), _ptr(o_idx), _ptr(o_lpl),
                                       _ptr(o_qo)))
    return o_ind, o_idx[:o_ind[-1]].copy(), o_lpl[:batch].copy(), o_qo


def timing_enable(plan: Plan, enable: bool = True):
    """pkv_timing_enable: record HIP events around every launch of this plan."""
    _check(_lib.pkv_timing_enable(plan.handle, 1 if enable else 0))


def timing_read(plan: Plan) -> dict:
    """pkv_timing_read: {kind: (summed ms, launches)} since the last read."""
    ms = (C.c_double * 4)()
    n = (C.c_int64 * 4)()
    _check(_lib.pkv_timing_read(plan.handle, ms, n))
    return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(TIMING_KINDS)}
