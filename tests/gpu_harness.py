"""Runs seeded workloads through the HIP library (via the Python binding) for
the GPU tests, the smoke check and the bench. Device buffers come from torch;
every step of the path runs in libpkv's kernels."""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
import torch

import paged_chunked_prefill_amd as pkv
import workloads as wl


def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage-format numpy array (bf16 bits as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def values_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def shape_of(w: wl.Workload) -> pkv.PkvShape:
    return pkv.make_shape(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.num_pages, w.dtype)


def torch_dtype(w: wl.Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


class DeviceCache:
    """K/V pools (NaN canaries in every unwritten slot) and the page table on the GPU."""

    def __init__(self, w: wl.Workload, device="cuda", page_table: Optional[np.ndarray] = None):
        self.w = w
        self.device = device
        shape = (w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
        self.k_pool = torch.full(shape, float("nan"), dtype=torch_dtype(w), device=device)
        self.v_pool = torch.full(shape, float("nan"), dtype=torch_dtype(w), device=device)
        pt = w.page_table if page_table is None else page_table
        self.page_table = torch.from_numpy(np.ascontiguousarray(pt, dtype=np.int32)).to(device)

    def append_step(self, step: wl.Workload, kv_storage=None, decode_splits: int = 0, num_cus: int = 0):
        """Append the step's chunk K/V (generated, or given in storage format)."""
        plan = pkv.build_extend_metadata(step.prefix_lens, step.chunk_lens, shape_of(step), step.window,
                                         decode_splits, device=self.device, num_cus=num_cus)
        if plan.plan.total_q == 0:
            return plan
        if kv_storage is None:
            kn, vn = self._gather_new_kv(step)
        else:
            kn, vn = (to_dev(x, step.dtype, self.device) for x in kv_storage)
        pkv.pkv_append(kn, vn, self.k_pool, self.v_pool, self.page_table, plan)
        return plan

    def _gather_new_kv(self, step: wl.Workload):
        """Chunk K/V of every request, uploaded request by request (no host copy of the whole batch)."""
        shp = (step.total_q, step.num_kv_heads, step.head_dim)
        kn = torch.empty(shp, dtype=torch_dtype(step), device=self.device)
        vn = torch.empty(shp, dtype=torch_dtype(step), device=self.device)
        row = 0
        for b in range(step.batch):
            L = int(step.chunk_lens[b])
            if L == 0:
                continue
            k, v = step.chunk_kv(b, storage=True)
            kn[row:row + L] = to_dev(k, step.dtype, self.device)
            vn[row:row + L] = to_dev(v, step.dtype, self.device)
            row += L
        return kn, vn

    def fill_prefix(self, w: wl.Workload):
        """Write every request's cached prefix (positions 0..P_b-1) with pkv_append."""
        return self.append_step(w.prefix_step())


def run_attention(cache: DeviceCache, w: wl.Workload, decode_splits: Optional[int] = None, q: Optional[torch.Tensor] = None,
                  sm_scale: float = 0.0, plan=None, num_cus: int = 0):
    """Append the chunk (unless a plan is given) and run the attention; returns (out, plan).
    ``num_cus`` sizes the plan for that many compute units (0: the device's)."""
    splits = w.decode_splits if decode_splits is None else decode_splits
    if plan is None:
        plan = cache.append_step(w, decode_splits=splits, num_cus=num_cus)
    if q is None:
        q = upload_q(w, cache.device)
    out = pkv.paged_extend_attn(q, cache.k_pool, cache.v_pool, cache.page_table, plan, sm_scale=sm_scale)
    return out, plan


def upload_q(w: wl.Workload, device="cuda") -> torch.Tensor:
    q = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch_dtype(w), device=device)
    row = 0
    for b in range(w.batch):
        L = int(w.chunk_lens[b])
        if L:
            q[row:row + L] = to_dev(w.q_chunk(b, storage=True), w.dtype, device)
            row += L
    return q


def prefill_and_attend(w: wl.Workload, decode_splits: Optional[int] = None, device="cuda",
                       page_table: Optional[np.ndarray] = None):
    """Fresh cache: write prefixes, append the chunk, attend. Returns (out, cache, plan)."""
    cache = DeviceCache(w, device, page_table)
    cache.fill_prefix(w)
    out, plan = run_attention(cache, w, decode_splits)
    return out, cache, plan


def chunked_prefill(w_full: wl.Workload, chunks, device="cuda", decode_splits: int = 0, num_cus: int = 0,
                    q_full: Optional[torch.Tensor] = None):
    """Prefill one request chunk by chunk; returns the concatenated outputs and the cache.
    ``q_full`` ([prompt, Hq, D] on the device) replaces the workload's queries."""
    cache = DeviceCache(w_full, device)
    outs = []
    pos = 0
    for step in wl.chunked_steps(w_full, chunks):
        L = int(step.chunk_lens[0])
        q = None if q_full is None else q_full[pos:pos + L].contiguous()
        out, _ = run_attention(cache, step, decode_splits, q=q, num_cus=num_cus)
        outs.append(out)
        pos += L
    torch.cuda.synchronize()
    return torch.cat(outs, 0), cache


def spare_page_pools(cache, spare: int = 16, k_fill: float = 1.0, v_fill: float = 16384.0):
    """Pools of the cache's declared page count followed by `spare` more pages of
    finite sentinels, returned as views of the declared size: a page id just
    past the declared pool stays inside the allocation, so a guard that failed
    to stop it would read (or write) the sentinels, never unmapped memory."""
    views = []
    for pool, fill in ((cache.k_pool, k_fill), (cache.v_pool, v_fill)):
        n = pool.shape[0]
        big = torch.full((n + spare,) + tuple(pool.shape[1:]), fill, dtype=pool.dtype, device=pool.device)
        big[:n].copy_(pool)
        views.append((big, big[:n]))
    return views
