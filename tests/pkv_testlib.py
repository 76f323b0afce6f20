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
