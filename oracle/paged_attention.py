"""CPU oracle for paged extend attention in chunked prefill.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or runs this
module; only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` do. It shares no code with the HIP path.

What it computes, from the pages:

* AReno PR #642, "What does this PR do?": when a prompt is prefilled in
  several chunks, each query of a later chunk attends to the request's cached
  prefix *and* its own chunk; the causal mask is aligned bottom-right, so
  query i of a chunk that follows a prefix of P tokens sees key positions
  0..P+i. Prefix and total-KV lengths travel with the batch metadata; new
  chunk K/V continues inside the last partly filled page.
* AstrAI compare v1.3.12..925cbed, ``astrai/inference/core/cache.py``
  (``PagePool.bind_tasks``): ``kv_indptr`` is the exclusive prefix sum of the
  per-request total lengths, and the write slots of a prefill step are the
  page-table entries of positions ``start_pos .. seq_len-1``.
* Same page, ``csrc/tests/attn_paged_test.cu`` (CPU reference for paged
  prefill): query head h reads KV head h // (Hq/Hkv); the causal offset of a
  request is its total length minus its chunk length; the scale defaults to
  1/sqrt(D).

The arithmetic is written for a reader to check by eye: for every request,
gather its K/V through the page table, then for every chunk row take the set
of visible key positions, form scaled dot products, subtract the maximum,
exponentiate and take the weighted mean of the visible V rows. It is a plain
two-pass softmax, not the online form of the pages' references. Precision is
a parameter: float32 (the default, as the method statement fixes) or float64.

Readings where the pages are silent (each also listed in the design notes):
* Sliding window W > 0: a query at absolute position p sees p-W+1 .. p
  (W positions counting its own); W <= 0 means no window.
* A row with no visible key (unreachable for valid input, since a causal row
  always sees itself) yields 0, as the pages' GPU kernels do.
* A request with no new tokens (L = 0) is a no-op.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# metadata  (AstrAI compare, cache.py PagePool.bind_tasks; AReno PR #642)
# ---------------------------------------------------------------------------

def extend_metadata(prefix_lens: Sequence[int], chunk_lens: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """qo_indptr[b] = number of new tokens before request b; kv_indptr[b] = number
    of total KV tokens (prefix + chunk) before request b. Both have B+1 entries."""
    P = np.asarray(prefix_lens, dtype=np.int64)
    L = np.asarray(chunk_lens, dtype=np.int64)
    qo = np.zeros(len(L) + 1, np.int64)
    kv = np.zeros(len(L) + 1, np.int64)
    qo[1:] = np.cumsum(L)
    kv[1:] = np.cumsum(P + L)
    return qo.astype(np.int32), kv.astype(np.int32)


def _row(page_table: np.ndarray, req_pool_indices: Optional[np.ndarray], b: int) -> np.ndarray:
    return page_table[int(req_pool_indices[b]) if req_pool_indices is not None else b]


# ---------------------------------------------------------------------------
# KV append  (AReno PR #642: "continue prefill inside the last allocated KV page")
# ---------------------------------------------------------------------------

def append_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              page_table: np.ndarray, prefix_lens: Sequence[int], chunk_lens: Sequence[int],
              req_pool_indices: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with each new token's K/V written to its slot.

    Pools are [num_pages, page_size, Hkv, D]; the new rows are [total_q, Hkv, D]
    in request order. Token i of request b sits at absolute position P_b + i,
    i.e. in logical page (P_b+i)//ps at offset (P_b+i)%ps, so the first new
    token lands inside the last, partly filled page whenever P_b % ps != 0.
    Works on any element type: the values are copied, not converted."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    ps = k_pool.shape[1]
    qo, _ = extend_metadata(prefix_lens, chunk_lens)
    for b in range(len(chunk_lens)):
        pages = _row(page_table, req_pool_indices, b)
        for i in range(int(chunk_lens[b])):
            pos = int(prefix_lens[b]) + i
            page, off = int(pages[pos // ps]), pos % ps
            k_out[page, off] = k_new[qo[b] + i]
            v_out[page, off] = v_new[qo[b] + i]
    return k_out, v_out


def gather_kv(pool: np.ndarray, pages: np.ndarray, n: int) -> np.ndarray:
    """Logical positions 0..n-1 of one request, read through its page-table row.
    Never touches a slot at a position >= n."""
    ps = pool.shape[1]
    j = np.arange(n)
    return pool[pages[j // ps].astype(np.int64), j % ps]


# ---------------------------------------------------------------------------
# attention  (AReno PR #642; AstrAI compare, attn_paged_test.cu CPU reference)
# ---------------------------------------------------------------------------

def visible_range(pos: int, window: int) -> Tuple[int, int]:
    """Key positions seen by the query at absolute position ``pos``: [lo, hi)."""
    hi = pos + 1
    lo = 0 if window <= 0 else max(0, pos - window + 1)
    return lo, hi


def extend_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, page_table: np.ndarray,
                     prefix_lens: Sequence[int], chunk_lens: Sequence[int], window: int = 0,
                     sm_scale: Optional[float] = None, req_pool_indices: Optional[np.ndarray] = None,
                     dtype=np.float32, rows: Optional[Iterable[int]] = None, causal: bool = True,
                     mask: Optional[np.ndarray] = None) -> np.ndarray:
    """Attention output [total_q, Hq, D] for a ragged batch of chunks.

    ``q`` holds the chunk queries [total_q, Hq, D] in request order; the pools
    already contain every request's prefix and chunk K/V. ``rows`` restricts the
    work to those global token indices (other rows are left NaN), for sampled
    checks of large batches. ``causal=False`` (AstrAI compare,
    attn_paged_prefill with is_causal=False: no causal offset) lets every row
    see all N_b keys of its request, chunk rows after it included.

    ``mask`` (same page: a bool mask, True = keep, 2-D [batch, kv_len] or 4-D
    [batch, 1 or heads, 1 or q_len, kv_len]) is taken here as an array
    [B, Hm, Qm, Ks] with Hm in {1, Hq} and Qm in {1, >= max chunk length}
    (a size-1 axis is shared by every head or row; a 2-D mask is Hm = Qm = 1)
    and Ks >= N_b, indexed by chunk row i and absolute key position j; a key
    is visible if the mask keeps it *and* it is in the causal/window range."""
    q = np.asarray(q)
    total_q, hq, d = q.shape
    hkv = k_pool.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    scale = (1.0 / math.sqrt(d)) if (sm_scale is None or sm_scale <= 0) else float(sm_scale)
    scale = dtype(scale)
    qo, kvp = extend_metadata(prefix_lens, chunk_lens)
    want = None if rows is None else set(int(r) for r in rows)
    out = np.full((total_q, hq, d), np.nan if want is not None else 0, dtype)
    if want is not None:
        for r in want:
            out[r] = 0
    for b in range(len(chunk_lens)):
        P, L = int(prefix_lens[b]), int(chunk_lens[b])
        if L == 0:
            continue
        if want is not None and not any(qo[b] <= r < qo[b] + L for r in want):
            continue
        n = P + L
        pages = _row(page_table, req_pool_indices, b)
        K = gather_kv(k_pool, pages, n).astype(dtype)      # [N, Hkv, D]
        V = gather_kv(v_pool, pages, n).astype(dtype)
        for i in range(L):
            t = int(qo[b]) + i
            if want is not None and t not in want:
                continue
            lo, hi = visible_range(P + i, window) if causal else (0, n)
            if hi <= lo:
                continue                                    # no visible key -> 0
            if mask is None:
                for kvh in range(hkv):
                    heads = slice(kvh * group, (kvh + 1) * group)   # query heads h with h // G == kvh
                    qv = q[t, heads].astype(dtype)                # [G, D]
                    keys = K[lo:hi, kvh]                          # [n_vis, D]
                    vals = V[lo:hi, kvh]
                    s = (qv @ keys.T) * scale                     # scores, [G, n_vis]
                    e = np.exp(s - s.max(axis=1, keepdims=True))
                    out[t, heads] = (e @ vals) / e.sum(axis=1, keepdims=True)
                continue
            # explicit mask: the kept keys of the range, per query head
            mrow = i if mask.shape[2] > 1 else 0
            for h in range(hq):
                keep = np.nonzero(mask[b, h if mask.shape[1] > 1 else 0, mrow, lo:hi])[0] + lo
                if keep.size == 0:
                    continue                                # no visible key -> 0
                kvh = h // group
                qv = q[t, h].astype(dtype)
                s = (K[keep, kvh] @ qv) * scale
                e = np.exp(s - s.max())
                out[t, h] = (e @ V[keep, kvh]) / e.sum()
    return out
