"""Helpers shared by the tests: run a seeded workload through the CPU oracle,
and compare results with the parity rule |a - ref| <= atol + rtol*|ref|."""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

import oracle
import workloads as wl

# Tolerances of the parity rule (bf16 inputs with fp32 accumulation / fp32 inputs).
TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}


def oracle_pools(w: wl.Workload, pools: Optional[Tuple[np.ndarray, np.ndarray]] = None,
                 with_chunk: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Storage-format pools holding every request's prefix (and chunk) K/V, written
    by the oracle's own append: first the prefix as a chunk starting at 0, then
    the chunk at P. Slots never written keep the NaN canary."""
    if pools is None:
        kp, vp = w.empty_pool(), w.empty_pool()
    else:
        kp, vp = pools
    pre = w.prefix_step()
    if pre.total_q:
        kn, vn = pre.new_kv_all()
        kp, vp = oracle.append_kv(kp, vp, kn, vn, w.page_table, pre.prefix_lens, pre.chunk_lens)
    if with_chunk and w.total_q:
        kn, vn = w.new_kv_all()
        kp, vp = oracle.append_kv(kp, vp, kn, vn, w.page_table, w.prefix_lens, w.chunk_lens)
    return kp, vp


def oracle_out(w: wl.Workload, pools: Tuple[np.ndarray, np.ndarray], dtype=np.float32,
               rows: Optional[Sequence[int]] = None, sm_scale: Optional[float] = None,
               causal: bool = True, mask: Optional[np.ndarray] = None) -> np.ndarray:
    kp, vp = pools
    q = wl.values(w.q_all(), w.dtype)
    return oracle.extend_attention(q, wl.values(kp, w.dtype), wl.values(vp, w.dtype), w.page_table,
                                   w.prefix_lens, w.chunk_lens, window=w.window, sm_scale=sm_scale,
                                   dtype=dtype, rows=rows, causal=causal, mask=mask)


def parity_report(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))        # NaN in got counts as bad
    rel = err / np.maximum(np.abs(ref), 1e-30)
    return {"ok": not bool(bad.any()), "n_bad": int(bad.sum()),
            "max_abs": float(np.nanmax(err)) if err.size else 0.0,
            "max_rel": float(np.nanmax(np.where(np.abs(ref) > 1e-3, rel, 0))) if err.size else 0.0,
            "nan": int(np.isnan(got).sum())}


def assert_parity(got, ref, dtype: str, what: str = ""):
    atol, rtol = TOL[dtype]
    rep = parity_report(got, ref, atol, rtol)
    assert rep["ok"], f"{what}: parity failed {rep}"
    return rep


# ---------------------------------------------------------------------------
# full-size comparisons: the oracle, as it is, over row blocks on threads
# ---------------------------------------------------------------------------

def worker_threads() -> int:
    """Threads for the oracle's row blocks: the CPUs this process may use, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compact_request(w: wl.Workload, b: int) -> Tuple[wl.Workload, Tuple[np.ndarray, np.ndarray]]:
    """Request b of ``w`` on its own: a one-request workload whose page-table row
    is 0, 1, 2, ... and a pool holding its K/V (prefix and chunk, storage
    format) at positions 0..N_b-1 in order; slots past N_b hold the canary.
    A layout only (the oracle gathers it back through the page table)."""
    P, L = int(w.prefix_lens[b]), int(w.chunk_lens[b])
    n = P + L
    npg = (n + w.page_size - 1) // w.page_size
    one = wl.Workload(w.name, w.config_id, w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, npg,
                      w.window, np.array([P], np.int32), np.array([L], np.int32),
                      np.arange(npg, dtype=np.int32)[None], request_ids=np.array([w.rid(b)]),
                      data_scale=w.data_scale, zero_q=w.zero_q, ramp_v=w.ramp_v, ramp_v_step=w.ramp_v_step)
    pools = []
    for seq in w.kv_seq(b, storage=True):
        pool = one.empty_pool()
        pool.reshape(npg * w.page_size, w.num_kv_heads, w.head_dim)[:n] = seq
        pools.append(pool)
    return one, (pools[0], pools[1])


def oracle_rows_parallel(w: wl.Workload, b: int, rows: Optional[Sequence[int]] = None, dtype=np.float32,
                         block: int = 32, causal: bool = True) -> np.ndarray:
    """``oracle.extend_attention`` for chunk rows ``rows`` (0-based within
    request b's chunk; default all of them) of one request, run over blocks of
    rows on a thread pool with single-threaded BLAS. Each block is one call of
    the oracle as it is; the blocks only divide the rows between threads.
    Returns [len(rows), Hq, D]."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    one, (kp, vp) = compact_request(w, b)
    L = int(one.chunk_lens[0])
    rows = list(range(L)) if rows is None else [int(r) for r in rows]
    q = wl.values(one.q_all(), one.dtype)
    kf, vf = wl.values(kp, one.dtype), wl.values(vp, one.dtype)
    blocks = [rows[i:i + block] for i in range(0, len(rows), block)]

    def run(rs):
        return oracle.extend_attention(q, kf, vf, one.page_table, one.prefix_lens, one.chunk_lens,
                                       window=one.window, dtype=dtype, rows=rs, causal=causal)[rs]

    with threadpool_limits(1), ThreadPoolExecutor(worker_threads()) as ex:
        parts = list(ex.map(run, blocks))
    return np.concatenate(parts, 0) if parts else np.zeros((0, w.num_q_heads, w.head_dim), dtype)
