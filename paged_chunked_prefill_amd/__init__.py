"""Python binding of libpkv: paged extend attention for chunked prefill on
MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels
(include/pkv.h documents the C ABI). PyTorch supplies device memory and the
stream. The functions carry the C names:

  build_extend_metadata(prefix_lens, chunk_lens, shape, window, decode_splits, device)
  pkv_append(k_new, v_new, k_pool, v_pool, page_table, plan)
  pkv_rope_append(q, k_new, v_new, rope_table, k_pool, v_pool, page_table, plan)
  paged_extend_attn(q, k_pool, v_pool, page_table, plan, out=None, ...)
  paged_extend_attn_masked(q, k_pool, v_pool, page_table, plan, mask, out=None, ...)
  paged_extend_attn_append(q, k_new, v_new, k_pool, v_pool, page_table, plan, out=None, ...)

There is no fallback: if libpkv.so is missing, importing this package
raises ImportError.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import _abi
from ._abi import (PKV_DTYPE_BF16, PKV_DTYPE_FP32, PKV_ERR_HIP, PKV_ERR_INVALID_ARGUMENT,  # noqa: F401
                   PKV_FLAG_NON_CAUSAL,
                   PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_MAX_SPLITS, PKV_NOALLOC_SCRATCH_BYTES, PKV_OK,
                   PKV_STATUS_BAD_PAGE, PkvPlan, PkvShape)

_lib = _abi.load()


def lib() -> ctypes.CDLL:
    return _lib


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def _check(status: int, what: str):
    if status != PKV_OK:
        raise PkvError(status, f"{what}: {_lib.pkv_last_error().decode(errors='replace')}")


def _dtype_code(dtype) -> int:
    name = str(dtype)
    if name in ("bf16", "torch.bfloat16", "bfloat16"):
        return PKV_DTYPE_BF16
    if name in ("fp32", "torch.float32", "float32"):
        return PKV_DTYPE_FP32
    if isinstance(dtype, int):
        return dtype
    raise ValueError(f"unsupported dtype {dtype}")


def make_shape(num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int,
               dtype="bf16") -> PkvShape:
    return PkvShape(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, _dtype_code(dtype))


def _i32(a: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _align256(x: int) -> int:
    return (x + 255) & ~255


# Work-list entry as laid out by the library (read back only by tests).
WORK_ITEM_DTYPE = np.dtype([("req", "<i4"), ("head_split", "<i4"), ("tok0", "<i4"), ("pos0", "<i4"),
                            ("q_count", "<i4"), ("kv_begin", "<i4"), ("kv_end", "<i4"), ("part_row", "<i4")])
SPLIT_BITS = 8
# Decoded view: the packed fields plus KV head, split and the tile's first chunk token.
WORK_ITEM_VIEW = np.dtype(WORK_ITEM_DTYPE.descr + [("kv_head", "<i4"), ("split", "<i4"), ("q_begin", "<i4"),
                                                  ("position", "<i4")])


def extend_metadata_size(prefix_lens, chunk_lens, shape: PkvShape, window: int = 0, decode_splits: int = 0,
                         causal: bool = True, num_cus: int = 0):
    P, L = _i32(prefix_lens), _i32(chunk_lens)
    mb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.pkv_extend_metadata_size_ex(len(L), _ptr(P), _ptr(L), ctypes.byref(shape), int(window),
                                            0 if causal else PKV_FLAG_NON_CAUSAL, int(decode_splits), int(num_cus),
                                            ctypes.byref(mb), ctypes.byref(wb)), "pkv_extend_metadata_size_ex")
    return mb.value, wb.value


class ExtendPlan:
    """A built step plan plus the buffers it points into (kept alive here)."""

    def __init__(self, plan: PkvPlan, shape: PkvShape, meta_host, meta_dev, prefix_lens, chunk_lens):
        self.plan = plan
        self.shape = shape
        self.meta_host = meta_host
        self.meta_dev = meta_dev
        self.prefix_lens = prefix_lens
        self.chunk_lens = chunk_lens
        self._workspace = None

    def __getattr__(self, name):
        return getattr(self.plan, name)

    def workspace(self):
        """A device buffer of the plan's workspace size (allocated once)."""
        import torch
        if self.plan.workspace_bytes == 0:
            return None
        if self._workspace is None or self._workspace.numel() < self.plan.workspace_bytes:
            self._workspace = torch.empty(self.plan.workspace_bytes, dtype=torch.uint8, device=self.meta_dev.device)
        return self._workspace

    def host_sections(self) -> dict:
        """Decode the host copy of the metadata (for inspection and tests)."""
        b, ni, ns = self.plan.batch, self.plan.n_items, self.plan.n_split_rows
        raw = self.meta_host.numpy() if hasattr(self.meta_host, "numpy") else self.meta_host
        raw = np.asarray(raw).view(np.uint8)
        off, out = 0, {}
        for name, count, dt in (("qo_indptr", b + 1, np.int32), ("kv_indptr", b + 1, np.int32),
                                ("prefix_lens", b, np.int32), ("items", ni, WORK_ITEM_DTYPE),
                                ("split_rows", 2 * ns, np.int32), ("status", 1, np.int32)):
            nbytes = np.dtype(dt).itemsize * count
            out[name] = raw[off:off + nbytes].view(dt).copy()
            off = _align256(off + nbytes)
        out["split_rows"] = out["split_rows"].reshape(-1, 2)
        # "items": the work items in dispatch order ("position" = workgroup index);
        # "padding": the empty items (q_count 0) that even out the XCD lists of a
        # stream plan, which the kernels skip
        raw_all = out["items"]
        real = raw_all["q_count"] > 0
        raw_items, items = raw_all[real], np.zeros(int(real.sum()), WORK_ITEM_VIEW)
        for f in WORK_ITEM_DTYPE.names:
            items[f] = raw_items[f]
        items["kv_head"] = raw_items["head_split"] >> (2 * SPLIT_BITS)
        items["split"] = raw_items["head_split"] & ((1 << SPLIT_BITS) - 1)
        items["q_begin"] = raw_items["tok0"] - out["qo_indptr"][raw_items["req"]]
        items["position"] = np.nonzero(real)[0]
        out["items"] = items
        out["padding"] = raw_all[~real]
        return out


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def build_extend_metadata(prefix_lens, chunk_lens, shape: PkvShape, window: int = 0, decode_splits: int = 0,
                          device=None, stream=None, meta_host=None, meta_dev=None, causal: bool = True,
                          num_cus: int = 0) -> ExtendPlan:
    """Plan one step. ``device=None`` plans on the host only (no GPU work).
    ``meta_host`` (pinned uint8 tensor) and ``meta_dev`` (device uint8 tensor)
    may be given to reuse buffers; the host one must not be rewritten before
    the copy enqueued here has run. ``causal=False`` plans with
    PKV_FLAG_NON_CAUSAL: every row sees its whole request. ``num_cus`` sizes
    the work list for that many compute units (0: the current device's)."""
    P, L = _i32(prefix_lens), _i32(chunk_lens)
    plan = PkvPlan()

    def call(host_ptr, host_bytes, dev_ptr, dev_bytes, st):
        return _check(_lib.build_extend_metadata_ex(len(L), _ptr(P), _ptr(L), ctypes.byref(shape), int(window),
                                                    0 if causal else PKV_FLAG_NON_CAUSAL, int(decode_splits),
                                                    int(num_cus), host_ptr, host_bytes, dev_ptr, dev_bytes,
                                                    ctypes.byref(plan), st), "build_extend_metadata_ex")

    if meta_host is not None and meta_dev is not None:
        call(ctypes.c_void_p(meta_host.data_ptr()), meta_host.numel(), ctypes.c_void_p(meta_dev.data_ptr()),
             meta_dev.numel(), _stream_handle(stream, meta_dev.device))
        return ExtendPlan(plan, shape, meta_host, meta_dev, P, L)
    meta_bytes, _ = extend_metadata_size(P, L, shape, window, decode_splits, causal, num_cus)
    if device is None:
        host = np.zeros(meta_bytes, np.uint8)
        call(_ptr(host), meta_bytes, None, 0, None)
        return ExtendPlan(plan, shape, host, None, P, L)
    import torch
    device = torch.device(device)
    host = torch.empty(meta_bytes, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(meta_bytes, dtype=torch.uint8, device=device)
    call(ctypes.c_void_p(host.data_ptr()), meta_bytes, ctypes.c_void_p(dev.data_ptr()), meta_bytes,
         _stream_handle(stream, device))
    return ExtendPlan(plan, shape, host, dev, P, L)


def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == PKV_DTYPE_BF16 else torch.float32


def _expect(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _check_tables(page_table, plan: ExtendPlan, req_pool_indices):
    """Types and shapes only: reading device values here would synchronise the
    stream on every call (and could not be captured into a graph). The values
    of req_pool_indices must be rows of page_table (check_req_pool_indices
    checks a host copy)."""
    import torch
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 [rows, stride] tensor")
    rows = page_table.shape[0]
    if req_pool_indices is None:
        if rows < plan.plan.batch:
            raise ValueError("page_table has fewer rows than requests")
    elif req_pool_indices.dtype != torch.int32 or req_pool_indices.numel() != plan.plan.batch \
            or not req_pool_indices.is_contiguous() or req_pool_indices.device != page_table.device:
        raise ValueError("req_pool_indices must be a contiguous int32 [batch] tensor on the page table's device")


def check_req_pool_indices(req_pool_indices_host, page_table_rows: int, batch: int) -> None:
    """Host-side check of request-pool row indices before they are uploaded:
    int32-representable, one per request, each a row of the page table."""
    r = np.asarray(req_pool_indices_host)
    if r.shape != (batch,) or r.size and (r.min() < 0 or r.max() >= page_table_rows):
        raise ValueError(f"req_pool_indices must hold {batch} rows of a {page_table_rows}-row page table")


def _pool_shape(s: PkvShape):
    return (s.num_pages, s.page_size, s.num_kv_heads, s.head_dim)


def pkv_append(k_new, v_new, k_pool, v_pool, page_table, plan: ExtendPlan, req_pool_indices=None, stream=None):
    """Write the chunk's K/V rows ([total_q, Hkv, D]) into their page slots."""
    s = plan.shape
    dt = _torch_dtype(s.dtype)
    tq = plan.plan.total_q
    _expect(k_new, (tq, s.num_kv_heads, s.head_dim), dt, "k_new")
    _expect(v_new, (tq, s.num_kv_heads, s.head_dim), dt, "v_new")
    _expect(k_pool, _pool_shape(s), dt, "k_pool")
    _expect(v_pool, _pool_shape(s), dt, "v_pool")
    _check_tables(page_table, plan, req_pool_indices)
    _check(_lib.pkv_append(ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
                           ctypes.c_void_p(k_pool.data_ptr()), ctypes.c_void_p(v_pool.data_ptr()),
                           ctypes.c_void_p(page_table.data_ptr()), page_table.shape[1],
                           ctypes.c_void_p(req_pool_indices.data_ptr()) if req_pool_indices is not None else None,
                           ctypes.byref(plan.plan), ctypes.byref(s), _stream_handle(stream, k_pool.device)),
           "pkv_append")


def pkv_rope_append(q, k_new, v_new, rope_table, k_pool, v_pool, page_table, plan: ExtendPlan, q_out=None,
                    req_pool_indices=None, stream=None):
    """Rotate the chunk's q and k rows at their absolute positions with
    ``rope_table`` (float32 [table_len, D/2, 2] = cos, sin) and write rotated K
    and V into their page slots. Returns q_out (a new tensor unless given;
    pass q itself to rotate in place)."""
    import torch
    s = plan.shape
    dt = _torch_dtype(s.dtype)
    tq = plan.plan.total_q
    _expect(q, (tq, s.num_q_heads, s.head_dim), dt, "q")
    _expect(k_new, (tq, s.num_kv_heads, s.head_dim), dt, "k_new")
    _expect(v_new, (tq, s.num_kv_heads, s.head_dim), dt, "v_new")
    _expect(k_pool, _pool_shape(s), dt, "k_pool")
    _expect(v_pool, _pool_shape(s), dt, "v_pool")
    if rope_table.dtype != torch.float32 or rope_table.dim() != 3 or tuple(rope_table.shape[1:]) != (s.head_dim // 2, 2) \
            or not rope_table.is_contiguous() or rope_table.device != q.device:
        raise ValueError(f"rope_table: expected contiguous float32 [n, {s.head_dim // 2}, 2] on {q.device}, got "
                         f"{rope_table.dtype} {tuple(rope_table.shape)} on {rope_table.device}")
    if q_out is None:
        q_out = torch.empty_like(q)
    _expect(q_out, (tq, s.num_q_heads, s.head_dim), dt, "q_out")
    _check_tables(page_table, plan, req_pool_indices)
    _check(_lib.pkv_rope_append(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q_out.data_ptr()),
                                ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
                                ctypes.c_void_p(rope_table.data_ptr()), rope_table.shape[0],
                                ctypes.c_void_p(k_pool.data_ptr()), ctypes.c_void_p(v_pool.data_ptr()),
                                ctypes.c_void_p(page_table.data_ptr()), page_table.shape[1],
                                ctypes.c_void_p(req_pool_indices.data_ptr()) if req_pool_indices is not None else None,
                                ctypes.byref(plan.plan), ctypes.byref(s), _stream_handle(stream, k_pool.device)),
           "pkv_rope_append")
    return q_out


def paged_extend_attn(q, k_pool, v_pool, page_table, plan: ExtendPlan, out=None, window: Optional[int] = None,
                      sm_scale: float = 0.0, req_pool_indices=None, qo_indptr=None, kv_indptr=None,
                      prefix_lens=None, workspace=None, stream=None):
    """Attention of every chunk row over its request's cached prefix + chunk."""
    import torch
    s = plan.shape
    dt = _torch_dtype(s.dtype)
    tq = plan.plan.total_q
    _expect(q, (tq, s.num_q_heads, s.head_dim), dt, "q")
    _expect(k_pool, _pool_shape(s), dt, "k_pool")
    _expect(v_pool, _pool_shape(s), dt, "v_pool")
    _check_tables(page_table, plan, req_pool_indices)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, (tq, s.num_q_heads, s.head_dim), dt, "out")
    if workspace is None:
        workspace = plan.workspace()
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    opt = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    _check(_lib.paged_extend_attn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_pool.data_ptr()),
                                  ctypes.c_void_p(v_pool.data_ptr()), ctypes.c_void_p(page_table.data_ptr()),
                                  page_table.shape[1], opt(req_pool_indices), opt(qo_indptr), opt(kv_indptr),
                                  opt(prefix_lens), plan.plan.window if window is None else int(window),
                                  float(sm_scale), ctypes.byref(plan.plan), ctypes.byref(s),
                                  ctypes.c_void_p(out.data_ptr()), ws_ptr, ws_bytes,
                                  _stream_handle(stream, q.device)), "paged_extend_attn")
    return out


def paged_extend_attn_append(q, k_new, v_new, k_pool, v_pool, page_table, plan: ExtendPlan, out=None,
                             window: Optional[int] = None, sm_scale: float = 0.0, req_pool_indices=None,
                             workspace=None, stream=None):
    """pkv_append of the chunk's K/V rows ([total_q, Hkv, D]) and the attention
    over the result, in one call (one attention launch for bf16)."""
    import torch
    s = plan.shape
    dt = _torch_dtype(s.dtype)
    tq = plan.plan.total_q
    _expect(q, (tq, s.num_q_heads, s.head_dim), dt, "q")
    _expect(k_new, (tq, s.num_kv_heads, s.head_dim), dt, "k_new")
    _expect(v_new, (tq, s.num_kv_heads, s.head_dim), dt, "v_new")
    _expect(k_pool, _pool_shape(s), dt, "k_pool")
    _expect(v_pool, _pool_shape(s), dt, "v_pool")
    _check_tables(page_table, plan, req_pool_indices)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, (tq, s.num_q_heads, s.head_dim), dt, "out")
    if workspace is None:
        workspace = plan.workspace()
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.paged_extend_attn_append(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(v_new.data_ptr()),
        ctypes.c_void_p(k_pool.data_ptr()), ctypes.c_void_p(v_pool.data_ptr()),
        ctypes.c_void_p(page_table.data_ptr()), page_table.shape[1],
        ctypes.c_void_p(req_pool_indices.data_ptr()) if req_pool_indices is not None else None,
        plan.plan.window if window is None else int(window), float(sm_scale), ctypes.byref(plan.plan),
        ctypes.byref(s), ctypes.c_void_p(out.data_ptr()), ws_ptr, ws_bytes, _stream_handle(stream, q.device)),
        "paged_extend_attn_append")
    return out


def paged_extend_attn_masked(q, k_pool, v_pool, page_table, plan: ExtendPlan, mask, out=None,
                             window: Optional[int] = None, sm_scale: float = 0.0, req_pool_indices=None,
                             workspace=None, stream=None):
    """paged_extend_attn with an explicit keep-mask: a bool or uint8 device
    tensor [B, 1 or Hq, 1 or >= max_q_len, Ks] (Ks >= max_kv_len, a multiple
    of 4), contiguous; nonzero keeps the (chunk row, absolute key) pair."""
    import torch
    s = plan.shape
    dt = _torch_dtype(s.dtype)
    tq = plan.plan.total_q
    _expect(q, (tq, s.num_q_heads, s.head_dim), dt, "q")
    _expect(k_pool, _pool_shape(s), dt, "k_pool")
    _expect(v_pool, _pool_shape(s), dt, "v_pool")
    _check_tables(page_table, plan, req_pool_indices)
    if mask.dtype not in (torch.bool, torch.uint8) or mask.dim() != 4 or not mask.is_contiguous() \
            or mask.shape[0] != plan.plan.batch or mask.device != q.device:
        raise ValueError(f"mask: expected a contiguous bool/uint8 [{plan.plan.batch}, Hm, Qm, Ks] tensor on "
                         f"{q.device}, got {mask.dtype} {tuple(mask.shape)} on {mask.device}")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, (tq, s.num_q_heads, s.head_dim), dt, "out")
    if workspace is None:
        workspace = plan.workspace()
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    opt = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    _check(_lib.paged_extend_attn_masked(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_pool.data_ptr()),
                                         ctypes.c_void_p(v_pool.data_ptr()), ctypes.c_void_p(page_table.data_ptr()),
                                         page_table.shape[1], opt(req_pool_indices), None, None, None,
                                         plan.plan.window if window is None else int(window), float(sm_scale),
                                         ctypes.c_void_p(mask.data_ptr()), mask.shape[1], mask.shape[2],
                                         mask.shape[3], ctypes.byref(plan.plan), ctypes.byref(s),
                                         ctypes.c_void_p(out.data_ptr()), ws_ptr, ws_bytes,
                                         _stream_handle(stream, q.device)), "paged_extend_attn_masked")
    return out


def paged_extend_attn_noalloc(q, k_pool, v_pool, page_table, plan: ExtendPlan, out, window: Optional[int] = None,
                              sm_scale: float = 0.0, req_pool_indices=None, stream=None):
    """paged_extend_attn with the split partials in the library's static
    per-device scratch (no workspace, nothing allocated; ``out`` must be given).
    Calls that overlap in time on one device race on that scratch."""
    s = plan.shape
    dt = _torch_dtype(s.dtype)
    tq = plan.plan.total_q
    _expect(q, (tq, s.num_q_heads, s.head_dim), dt, "q")
    _expect(k_pool, _pool_shape(s), dt, "k_pool")
    _expect(v_pool, _pool_shape(s), dt, "v_pool")
    _check_tables(page_table, plan, req_pool_indices)
    _expect(out, (tq, s.num_q_heads, s.head_dim), dt, "out")
    opt = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    _check(_lib.paged_extend_attn_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_pool.data_ptr()),
                                          ctypes.c_void_p(v_pool.data_ptr()), ctypes.c_void_p(page_table.data_ptr()),
                                          page_table.shape[1], opt(req_pool_indices), None, None, None,
                                          plan.plan.window if window is None else int(window), float(sm_scale),
                                          ctypes.byref(plan.plan), ctypes.byref(s), ctypes.c_void_p(out.data_ptr()),
                                          _stream_handle(stream, q.device)), "paged_extend_attn_noalloc")
    return out


def read_status(plan: ExtendPlan, stream=None) -> int:
    st = ctypes.c_int32()
    _check(_lib.pkv_read_status(ctypes.byref(plan.plan), ctypes.byref(st),
                                _stream_handle(stream, plan.meta_dev.device)), "pkv_read_status")
    return st.value


def device_supported(device: int = 0) -> bool:
    r = _lib.pkv_device_supported(int(device))
    if r < 0:
        _check(r, "pkv_device_supported")
    return bool(r)
